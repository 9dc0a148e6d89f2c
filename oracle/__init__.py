"""CPU oracle (test infrastructure): a plain float64 reference of one SparSTAR scale.

Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from .sparstar_oracle import *  # noqa: F401,F403
