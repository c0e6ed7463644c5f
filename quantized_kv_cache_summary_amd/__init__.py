"""Importance-based sparse decode attention over a paged, optionally low-bit KV cache, for MI355X.

The compute path is the HIP library ``libkvsparse.so`` (hand-written gfx950
kernels behind the C ABI in ``include/kvsparse.h``); ``kvsparse`` is its thin
ctypes binding.  Importing this package loads nothing: the binding loads the
library on first use and raises if it has not been built.
"""

__all__ = ["kvsparse", "workloads"]
