"""SparSTAR dynamic block-sparse attention for one expensive scale, on MI355X (gfx950).

The compute lives in ``libsparstar.so`` (hand-written HIP kernels behind a
C ABI, declared in include/sparstar.h); :mod:`.sparstar` is the thin ctypes
binding over it.  :mod:`.inputs` draws seeded synthetic Q/K/V.  Importing the
package does not load the library; the binding loads it on first use and
raises if it is missing.
"""

__all__ = ["inputs", "sparstar"]
