"""Paged attention, fp64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

ARTICLE §2.3 (PagedAttention kernel): for every query token, find the K/V
blocks of its sequence through ``block_tables``, up to the sequence's
``context_lens``, and compute attention over them (scores within a block,
accumulated across blocks).  The accumulation order does not change the
exact result, which is ordinary softmax attention over the gathered keys:

    z_p   = sm_scale * <q, K_p>                 for the admissible keys p
    w_p   = exp(z_p - max z) / sum_p' exp(z_p' - max z)
    out   = sum_p w_p V_p

Admissible keys:
* decode (one query per sequence, the sequence's newest token): all
  positions ``0 .. L-1`` where L is the context length and already counts the
  query's own token (its K/V are written before attention is computed);
* a chunked-prefill slice (LESSON, "Chunked prefill": a long prompt is cut
  into fixed 512-token slices, each scheduled as one unit): the query at
  absolute position ``P0 + i`` sees positions ``0 .. P0 + i`` inclusive
  (causal), where ``P0`` is the slice's first position.

Readings where the texts are silent:
* grouped-query heads: the pools are shaped with the KV head count; query
  head h reads KV head ``h // (H_q / H_kv)`` (contiguous groups);
* ``sm_scale`` is the float32 value handed to the kernel (normally
  ``1/sqrt(D)`` rounded to float32), used here exactly, in fp64;
* fp8 caches: a stored code decodes to ``table_value * scale`` in fp64
  (exact), with separate per-tensor scales for K and V.

Every step is fp64; the gather is a plain index loop over positions, and the
contractions are numpy matrix products (library primitives).
"""
from __future__ import annotations

import numpy as np

from . import codecs


def kv_head_of(h: int, h_q: int, h_kv: int) -> int:
    return h // (h_q // h_kv)


def gather(k_cache, v_cache, table, length: int, kv_head: int, cache_dtype: str,
           k_scale: float = 1.0, v_scale: float = 1.0):
    """Keys and values of positions 0..length-1 of one sequence and KV head,
    fetched through the block table, as fp64 [length, D] arrays."""
    bs = k_cache.shape[3]
    d = v_cache.shape[2]
    pos = np.arange(length)
    blocks = np.asarray(table, dtype=np.int64)[pos // bs]
    if length and blocks.min() < 0:
        raise ValueError("block table shorter than the context")
    offs = pos % bs
    k_raw = k_cache[blocks, kv_head, :, offs, :].reshape(length, d)   # [L, D]
    v_raw = v_cache[blocks, kv_head, :, offs]            # [L, D]
    k = codecs.decode(k_raw, cache_dtype)
    v = codecs.decode(v_raw, cache_dtype)
    if cache_dtype == "fp8":
        k = k * float(np.float32(k_scale))
        v = v * float(np.float32(v_scale))
    assert k.shape == (length, d)
    return k, v


def softmax_attention(q, k, v, sm_scale: float, limits=None):
    """q [n, D], k/v [L, D] fp64.  Row i attends keys 0 .. limits[i]-1
    (all L when ``limits`` is None).  Returns [n, D] fp64."""
    z = (q @ k.T) * float(np.float32(sm_scale))          # [n, L]
    if limits is not None:
        cols = np.arange(k.shape[0])[None, :]
        z = np.where(cols < np.asarray(limits)[:, None], z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    w = e / e.sum(axis=1, keepdims=True)
    return w @ v


def decode(q, k_cache, v_cache, tables, context_lens, h_kv: int, sm_scale: float,
           cache_dtype: str, k_scale=1.0, v_scale=1.0, pairs=None):
    """Decode attention.  q: [S, H_q, D] fp64; tables: [S, max_blocks];
    returns [S, H_q, D] fp64 (rows not in ``pairs`` left NaN when a subset of
    (sequence, query head) pairs is requested)."""
    s_n, h_q, d = q.shape
    out = np.full((s_n, h_q, d), np.nan)
    g = h_q // h_kv
    want = None if pairs is None else {(int(a), int(b)) for a, b in pairs}
    for s in range(s_n):
        L = int(context_lens[s])
        if L <= 0:
            raise ValueError("decode needs a context of at least one token")
        for kh in range(h_kv):
            heads = [h for h in range(kh * g, (kh + 1) * g) if want is None or (s, h) in want]
            if not heads:
                continue
            k, v = gather(k_cache, v_cache, tables[s], L, kh, cache_dtype, k_scale, v_scale)
            out[s, heads] = softmax_attention(q[s, heads], k, v, sm_scale)
    return out


def prefill_chunk(q, start_pos: int, k_cache, v_cache, table, h_kv: int, sm_scale: float,
                  cache_dtype: str, k_scale=1.0, v_scale=1.0, rows=None):
    """Causal attention of one prefill slice against its paged prefix.

    q: [n, H_q, D] fp64 for positions start_pos .. start_pos+n-1.  The
    keys of positions 0 .. start_pos+n-1 must already be in the cache.
    ``rows`` optionally restricts the computation to a subset of query rows
    (others stay NaN).
    """
    n, h_q, d = q.shape
    g = h_q // h_kv
    out = np.full((n, h_q, d), np.nan)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    if len(rows) == 0:
        return out
    total = start_pos + int(rows.max()) + 1
    limits = start_pos + rows + 1
    for kh in range(h_kv):
        k, v = gather(k_cache, v_cache, table, total, kh, cache_dtype, k_scale, v_scale)
        for h in range(kh * g, (kh + 1) * g):
            out[rows, h] = softmax_attention(q[rows, h], k, v, sm_scale, limits)
    return out
