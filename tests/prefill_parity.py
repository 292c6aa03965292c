"""Prefill-slice runners for the parity tests: HIP library vs CPU oracle,
sharing only the ``workloads`` arrays."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_host_amd as pa
from paged_kv_cache_host_amd.engine import PagedKV, prefill_workspace, to_device_raw, to_host_raw
from oracle import allocator as oa
from oracle import attention as oat
from oracle import cache as oc
from oracle import codecs
from tests.parity import filled


def _slice_rows(w):
    offs = w.token_offsets()
    return np.concatenate([np.arange(offs[s] + a, offs[s] + a + n) for s, a, n in w.slices])


def hip_prefill_run(w, device="cuda", free_order=None):
    order = w.free_order if free_order is None else free_order
    kv = PagedKV(w.num_blocks, w.h_kv, w.d, w.cache_dtype, device, order, w.k_scale, w.v_scale)
    slots = []
    for s, P in enumerate(w.prompts.tolist()):
        pa.check(kv.create(s, int(P)))
        slots.append(kv.slots(s, 0, int(P)))
    slots = np.concatenate(slots).astype(np.int32)
    kv.write(to_device_raw(w.k_tok, w.kv_dtype, device), to_device_raw(w.v_tok, w.kv_dtype, device),
             torch.from_numpy(slots).to(device))
    seqs = [s for s, _, _ in w.slices]
    tables, _ = kv.pack(seqs, max(1, max(-(-int(P) // 16) for P in w.prompts)))
    rows = _slice_rows(w)
    q = to_device_raw(w.q_tok[rows], w.q_dtype, device)
    cu = np.concatenate([[0], np.cumsum([n for _, _, n in w.slices])]).astype(np.int32)
    start = np.array([a for _, a, _ in w.slices], dtype=np.int32)
    max_q = max(n for _, _, n in w.slices)
    max_ctx = max(a + n for _, a, n in w.slices)
    out_dt = torch.float32 if w.q_dtype == "f32" else torch.bfloat16
    out = filled((len(rows), w.h_q, w.d), out_dt, device)
    ws = prefill_workspace(len(w.slices), max_q, w.h_q, w.h_kv, w.d, max_ctx, device)
    kv.prefill(out, q, torch.from_numpy(cu).to(device), torch.from_numpy(start).to(device),
               torch.from_numpy(tables).to(device), max_q, max_ctx, w.sm_scale, ws)
    torch.cuda.synchronize()
    return {"out": to_host_raw(out, w.q_dtype), "tables": tables, "slots": slots, "kv": kv}


def oracle_prefill_run(w, rows_per_slice=None):
    """rows_per_slice: optional {slice index: array of query rows} to compute
    (others left NaN)."""
    pool = oa.BlockPool(w.num_blocks, 16, w.free_order.tolist())
    offs = w.token_offsets()
    kc, vc = oc.new_cache(w.num_blocks, w.h_kv, 16, w.d, w.cache_dtype)
    for s, P in enumerate(w.prompts.tolist()):
        assert pool.seq_create(s, int(P)) == oa.OK
        oc.cache_write(kc, vc, w.k_tok[offs[s]:offs[s + 1]], w.v_tok[offs[s]:offs[s + 1]],
                       pool.slots(s, 0, int(P)), w.kv_dtype, w.cache_dtype, w.k_scale, w.v_scale)
    outs = []
    for i, (s, a, n) in enumerate(w.slices):
        q = codecs.decode(w.q_tok[offs[s] + a: offs[s] + a + n], w.q_dtype)
        rows = None if rows_per_slice is None else rows_per_slice.get(i, np.array([], dtype=np.int64))
        outs.append(oat.prefill_chunk(q, a, kc, vc, pool.block_table(s), w.h_kv, w.sm_scale,
                                      w.cache_dtype, w.k_scale, w.v_scale, rows=rows))
    return {"out": np.concatenate(outs), "kc": kc, "vc": vc}
