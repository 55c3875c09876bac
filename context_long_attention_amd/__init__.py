"""One rank's share of context-parallel Pass-KV ring attention on AMD MI355X (gfx950).

The compute lives in ``libcpattn.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/cpattn.h``).  ``cpattn`` is the thin ctypes binding with
the same names; ``ring`` replays one rank's ring steps on one GPU.  Importing
this package loads nothing: the library is opened on first use and a missing
library is an error, never a fallback.
"""
__all__ = ["inputs", "cpattn", "ring"]
