"""CPU oracle (test infrastructure): a plain float64 reference of one SparSTAR scale.

Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
`oracle.retained_mass` holds the retained-attention-mass measures.
"""
from .sparstar_oracle import *  # noqa: F401,F403
from . import retained_mass  # noqa: F401
