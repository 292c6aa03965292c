"""Helpers for the GPU parity tests: run one workload through the HIP
library (via its C ABI binding) and, independently, through the CPU oracle.

The two runners share nothing but the workload arrays produced by
``workloads``: the HIP side uses libpa's pool, cache write and kernels; the
oracle side uses ``oracle``'s allocator, scatter and fp64 attention.
"""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_host_amd as pa
from paged_kv_cache_host_amd.engine import PagedKV, decode_workspace, prefill_workspace, to_device_raw, to_host_raw
from oracle import allocator as oa
from oracle import attention as oat
from oracle import cache as oc
from oracle import codecs
from tests.gate import SENTINEL, TOL, assert_close  # noqa: F401  (re-exported)


def out_to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    return codecs.decode(raw, dtype)


def filled(shape, dtype, device) -> torch.Tensor:
    """An output buffer holding the gate's sentinel in every element, so
    that rows no kernel writes fail the comparison."""
    return torch.full(shape, SENTINEL, dtype=dtype, device=device)


# -------------------------------------------------------------- decode -----

def hip_decode_run(w, device="cuda", free_order=None, reps=1):
    """Fill a fresh pool with the workload's K/V through pa_cache_write and
    run pa_decode.  Returns dict with host copies of the outputs, tables,
    slots and (optionally) the cache bytes."""
    order = w.free_order if free_order is None else free_order
    kv = PagedKV(w.num_blocks, w.h_kv, w.d, w.cache_dtype, device, order, w.k_scale, w.v_scale)
    S = w.num_seqs
    slots = []
    for s, L in enumerate(w.lengths.tolist()):
        pa.check(kv.create(s, int(L)))
        slots.append(kv.slots(s, 0, int(L)))
    slots = np.concatenate(slots).astype(np.int32)
    k_new = to_device_raw(w.k_tok, w.kv_dtype, device)
    v_new = to_device_raw(w.v_tok, w.kv_dtype, device)
    kv.write(k_new, v_new, torch.from_numpy(slots).to(device))
    del k_new, v_new
    tables, lens = kv.pack(list(range(S)))
    t_d = torch.from_numpy(tables).to(device)
    l_d = torch.from_numpy(lens).to(device)
    q = to_device_raw(w.q, w.q_dtype, device)
    out_dt = torch.float32 if w.q_dtype == "f32" else torch.bfloat16
    max_ctx = int(w.lengths.max())
    ws = decode_workspace(S, w.h_q, w.h_kv, w.d, max_ctx, device)
    outs = []
    for _ in range(reps):
        out = filled((S, w.h_q, w.d), out_dt, device)
        kv.decode(out, q, t_d, l_d, max_ctx, w.sm_scale, ws)
        outs.append(to_host_raw(out, w.q_dtype))
    torch.cuda.synchronize()
    res = {"outs": outs, "tables": tables, "lens": lens, "slots": slots, "kv": kv}
    return res


def oracle_decode_run(w, seqs=None, pairs=None):
    """Oracle side.  ``seqs``: only these sequences' tokens are scattered
    (the tables are still built for all, so that they can be compared);
    ``pairs``: (sequence, head) pairs to compute."""
    pool = oa.BlockPool(w.num_blocks, 16, w.free_order.tolist())
    offs = w.token_offsets()
    slots = []
    for s, L in enumerate(w.lengths.tolist()):
        assert pool.seq_create(s, int(L)) == oa.OK
        slots.append(pool.slots(s, 0, int(L)))
    kc, vc = oc.new_cache(w.num_blocks, w.h_kv, 16, w.d, w.cache_dtype)
    want = range(w.num_seqs) if seqs is None else seqs
    for s in want:
        a, b = offs[s], offs[s + 1]
        oc.cache_write(kc, vc, w.k_tok[a:b], w.v_tok[a:b], slots[s], w.kv_dtype, w.cache_dtype,
                       w.k_scale, w.v_scale)
    mb = max(-(-int(L) // 16) for L in w.lengths)
    tables, lens = pool.pack(range(w.num_seqs), mb)
    tables = np.array(tables, dtype=np.int32)
    lens = np.array(lens, dtype=np.int32)
    q = codecs.decode(w.q, w.q_dtype)
    if pairs is None and seqs is not None:
        pairs = [(s, h) for s in seqs for h in range(w.h_q)]
    out = oat.decode(q, kc, vc, tables, lens, w.h_kv, w.sm_scale, w.cache_dtype, w.k_scale,
                     w.v_scale, pairs)
    return {"out": out, "tables": tables, "lens": lens,
            "slots": np.concatenate([np.asarray(x, dtype=np.int32) for x in slots]), "kc": kc,
            "vc": vc}
