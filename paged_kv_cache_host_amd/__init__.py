"""Paged-attention hot path for AMD Instinct MI355X (gfx950).

The library ``libpa.so`` (C ABI in ``include/pa.h``) holds the host block
allocator and the HIP kernels; ``paged_kv_cache_host_amd._pa`` is its ctypes
binding, re-exported here under the C names.  The library is loaded on first
use of any of those names (so that ``paged_kv_cache_host_amd.build`` can run
before it exists); a missing library raises ImportError there.
"""
import importlib as _importlib


def __getattr__(name):
    if name.startswith("__"):
        raise AttributeError(name)
    _pa = _importlib.import_module("._pa", __name__)
    try:
        return getattr(_pa, name)
    except AttributeError:
        raise AttributeError(f"module {__name__!r} has no attribute {name!r}") from None
