"""Scatter of new K/V vectors into the paged cache (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

LESSON, "The Concept: PagedAttention as a virtual memory system": the K/V of
token position p of a sequence lives in physical block ``table[p // bs]`` at
offset ``p % bs``.  The flat slot ``table[p // bs] * bs + p % bs`` therefore
names one (block, offset) cell; writing a token means storing its K and V
vectors for every KV head in that cell.

Cache layout (the library's contract, per physical block ``b`` and KV head
``h``; ``x`` = elements per 16 bytes: 4 for fp32, 8 for bf16, 16 for fp8):
  K cache  [num_blocks][H_kv][D/x][bs][x]  -- key dims d..d+x-1 of the 16
                                              tokens of a block are adjacent
  V cache  [num_blocks][H_kv][D][bs]       -- a token's value is a column
The ARTICLE (§2.2) shapes both pools ``[num_blocks, block_size, num_heads,
head_dim]``; the order of the axes inside a pool is a layout choice that does
not change what is stored, only where.

Encoding of a stored element: identity when the new vectors already have the
cache's type; for the fp8 cache, ``e4m3_quantize(x, scale)`` (see codecs).
Slots below zero mean "skip this token".
"""
from __future__ import annotations

import numpy as np

from . import codecs


def chunk_elems(dtype: str) -> int:
    """Elements per 16-byte chunk of the K layout."""
    return 16 // np.dtype(codecs.storage_numpy_dtype(dtype)).itemsize


def new_cache(num_blocks: int, h_kv: int, bs: int, d: int, dtype: str):
    """Zero-filled K and V pools in storage dtype (ARTICLE §2.2 allocates
    the pools once, zero-initialised)."""
    nd = codecs.storage_numpy_dtype(dtype)
    x = chunk_elems(dtype)
    k = np.zeros((num_blocks, h_kv, d // x, bs, x), dtype=nd)
    v = np.zeros((num_blocks, h_kv, d, bs), dtype=nd)
    return k, v


def encode_for_cache(x_raw: np.ndarray, new_dtype: str, cache_dtype: str, scale: float):
    """Convert new vectors (raw storage of ``new_dtype``) to cache codes."""
    if new_dtype == cache_dtype:
        return np.asarray(x_raw, dtype=codecs.storage_numpy_dtype(cache_dtype))
    if new_dtype == "bf16" and cache_dtype == "fp8":
        x32 = codecs.bf16_decode(x_raw).astype(np.float32)      # exact
        return codecs.e4m3_quantize(x32, np.float32(scale))
    raise ValueError(f"unsupported conversion {new_dtype} -> {cache_dtype}")


def cache_write(k_cache, v_cache, k_new_raw, v_new_raw, slots, new_dtype, cache_dtype,
                k_scale=1.0, v_scale=1.0):
    """In-place scatter.  ``k_new_raw``, ``v_new_raw``: [n, H_kv, D] raw."""
    bs = k_cache.shape[3]
    h_kv, nchunk, x = k_cache.shape[1], k_cache.shape[2], k_cache.shape[4]
    kq = encode_for_cache(k_new_raw, new_dtype, cache_dtype, k_scale)
    vq = encode_for_cache(v_new_raw, new_dtype, cache_dtype, v_scale)
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    live = slots[keep]
    if len(np.unique(live)) != len(live):
        raise ValueError("slots of one write must be distinct")
    b, o = live // bs, live % bs
    k_cache[b, :, :, o, :] = kq[keep].reshape(-1, h_kv, nchunk, x)
    v_cache[b, :, :, o] = vq[keep]
