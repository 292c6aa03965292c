"""Paged-attention hot path for AMD Instinct MI355X (gfx950).

The library ``libpa.so`` (C ABI in ``include/pa.h``) holds the host block
allocator and the HIP kernels; ``paged_kv_cache_host_amd._pa`` is its ctypes
binding.  Importing the package loads the library and fails loudly if it has
not been built (``python -m paged_kv_cache_host_amd.build``).
"""
from . import _pa  # noqa: F401  (loads libpa.so)
from ._pa import *  # noqa: F401,F403
