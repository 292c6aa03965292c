"""Host orchestration of one attention layer's paged KV cache.

Thin layer over libpa: torch owns the device pools, work buffers and the
stream; every allocation decision is made by libpa's host pool and every
device step by its kernels.  Used by the benchmark, the parity tests and the
continuous-batching trace driver.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import _pa as pa

BLOCK = 16

_TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
_NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def to_device_raw(raw: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload a raw storage array (float32 / uint16 bf16 bits / uint8 fp8
    codes) as a torch tensor of the matching storage dtype."""
    raw = np.ascontiguousarray(raw)
    if dtype == "bf16":
        t = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(raw.astype(np.float32, copy=False))
    elif dtype == "fp8":
        t = torch.from_numpy(raw.astype(np.uint8, copy=False))
    else:
        raise ValueError(dtype)
    return t.to(device, non_blocking=False)


def to_host_raw(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    if dtype == "f32":
        return t.numpy()
    return t.numpy().astype(np.uint8, copy=False)


class PagedKV:
    """K/V pools of one layer on the device plus libpa's host block pool."""

    def __init__(self, num_blocks: int, h_kv: int, d: int, cache_dtype: str, device="cuda",
                 free_order=None, k_scale: float = 1.0, v_scale: float = 1.0):
        st, pool = pa.pa_pool_create(num_blocks, BLOCK, free_order)
        pa.check(st)
        self.pool = pool
        self.num_blocks = num_blocks
        self.h_kv = h_kv
        self.d = d
        self.cache_dtype = cache_dtype
        self.k_scale = float(k_scale)
        self.v_scale = float(v_scale)
        dt = _TORCH_STORAGE[cache_dtype]
        x = 16 // torch.empty((), dtype=dt).element_size()   # elements per 16-byte chunk
        self.k = torch.zeros((num_blocks, h_kv, d // x, BLOCK, x), dtype=dt, device=device)
        self.v = torch.zeros((num_blocks, h_kv, d, BLOCK), dtype=dt, device=device)

    def close(self):
        if self.pool is not None:
            pa.pa_pool_destroy(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # host allocator ---------------------------------------------------------
    def create(self, seq: int, n: int) -> int:
        return pa.pa_seq_create(self.pool, seq, n)

    def append(self, seq: int, n: int):
        return pa.pa_seq_append(self.pool, seq, n)

    def slots(self, seq: int, start: int, n: int) -> np.ndarray:
        st, s = pa.pa_seq_slots(self.pool, seq, start, n)
        pa.check(st)
        return s

    def release(self, seq: int) -> int:
        return pa.pa_seq_release(self.pool, seq)

    def pack(self, seqs, max_blocks: int | None = None, out_tables=None, out_lens=None):
        if max_blocks is None:
            lens = []
            for s in seqs:
                st, n = pa.pa_seq_length(self.pool, s)
                pa.check(st)
                lens.append(n)
            max_blocks = max(1, max(-(-n // BLOCK) for n in lens) if lens else 1)
        st, tables, lens = pa.pa_pack_batch(self.pool, seqs, max_blocks, out_tables, out_lens)
        pa.check(st)
        return tables, lens

    # device steps -------------------------------------------------------------
    def write(self, k_new: torch.Tensor, v_new: torch.Tensor, slots: torch.Tensor, stream=None):
        pa.check(pa.pa_cache_write(stream, k_new, v_new, slots, self.k, self.v, self.num_blocks,
                                   self.h_kv, self.d, BLOCK, self.k_scale, self.v_scale))

    def decode(self, out, q, tables, lens, max_context_len: int, sm_scale: float, ws=None,
               stream=None):
        pa.check(pa.pa_decode(stream, out, q, self.k, self.v, tables, lens, self.num_blocks,
                              self.h_kv, max_context_len, sm_scale, self.k_scale, self.v_scale,
                              ws))

    def prefill(self, out, q, cu_q_lens, start_pos, tables, max_q_len: int,
                max_context_len: int, sm_scale: float, ws=None, stream=None):
        pa.check(pa.pa_prefill_chunk(stream, out, q, cu_q_lens, start_pos, self.k, self.v, tables,
                                     self.num_blocks, self.h_kv, max_q_len, max_context_len,
                                     sm_scale, self.k_scale, self.v_scale, ws))

    def attend_varlen(self, out, q, cu_q_lens, seq_lens, n_decode: int, dec_tables, pf_tables,
                      max_q_len: int, max_decode_len: int, max_prefill_len: int,
                      sm_scale: float, bufs, stream=None):
        """Decode rows and prefill slices in one launch; bufs = varlen_buffers(...)."""
        counters, ws = bufs
        pa.check(pa.pa_attend_varlen(stream, out, q, cu_q_lens, seq_lens, n_decode, self.k,
                                     self.v, dec_tables, pf_tables, self.num_blocks, self.h_kv,
                                     max_q_len, max_decode_len, max_prefill_len, sm_scale,
                                     self.k_scale, self.v_scale, counters, ws))


def varlen_buffers(n_decode, n_prefill, h_q, h_kv, d, max_q_len, max_decode_len,
                   max_prefill_len, device="cuda"):
    """(counters, workspace) for pa_attend_varlen calls within these sizes:
    the counters zero-filled (every call leaves them zero), the workspace
    uninitialised (None when no call within the sizes needs one)."""
    nc = pa.pa_attend_varlen_counters(n_decode, n_prefill, h_q, h_kv, max_q_len)
    nb = pa.pa_attend_varlen_workspace_bytes(n_decode, n_prefill, h_q, h_kv, d, max_q_len,
                                             max_decode_len, max_prefill_len)
    counters = torch.zeros(max(nc, 2), dtype=torch.int32, device=device)
    ws = torch.empty(nb, dtype=torch.uint8, device=device) if nb > 0 else None
    return counters, ws


def decode_workspace(S, h_q, h_kv, d, max_context_len, device="cuda") -> torch.Tensor | None:
    """Zero-filled decode workspace (its work counters must start at zero;
    every call leaves them zero)."""
    n = pa.pa_decode_workspace_bytes(S, h_q, h_kv, d, max_context_len)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def prefill_workspace(n_chunks, max_q_len, h_q, h_kv, d, max_context_len, device="cuda"):
    n = pa.pa_prefill_workspace_bytes(n_chunks, max_q_len, h_q, h_kv, d, max_context_len)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def sm_scale_for(d: int) -> float:
    return float(np.float32(1.0) / np.float32(math.sqrt(d)))
