"""Runners for pa_attend_varlen parity (HIP library vs CPU oracle): a
mixed batch of decode rows and prefill slices, written into one cache, with
the device arguments of one fused call.  Shared by the GPU tests and
smoke(); only the ``workloads`` arrays are shared with the oracle side."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_host_amd as pa
import workloads
from paged_kv_cache_host_amd.engine import (PagedKV, decode_workspace, prefill_workspace,
                                            to_device_raw, to_host_raw, varlen_buffers)
from tests.parity import filled
from tests.prefill_parity import oracle_prefill_run

DEV = "cuda"


def mixed_batch(name, seed, decode_lens, prompts, slices, h_q=16, h_kv=2, d=128,
                cache_dtype="bf16"):
    """A PrefillWorkload whose first len(decode_lens) sequences are decode
    rows (one query at the last position of a context of that length) and
    whose further sequences are the prompts, attended by ``slices``
    (prompt index, start, n)."""
    n_dec = len(decode_lens)
    all_prompts = list(decode_lens) + list(prompts)
    all_slices = [(i, int(L) - 1, 1) for i, L in enumerate(decode_lens)]
    all_slices += [(n_dec + s, a, n) for s, a, n in slices]
    return workloads.prefill_workload(name, seed, prompts=all_prompts, slices=all_slices, h_q=h_q,
                                      h_kv=h_kv, d=d, cache_dtype=cache_dtype), n_dec


class Batch:
    """The cache written with every sequence's tokens, and the device
    arguments of the batch (q rows, cu_q_lens, seq_lens, tables)."""

    def __init__(self, w, n_dec):
        self.w, self.n_dec = w, n_dec
        self.kv = PagedKV(w.num_blocks, w.h_kv, w.d, w.cache_dtype, DEV, w.free_order, w.k_scale,
                          w.v_scale)
        slots = []
        for s, P in enumerate(w.prompts.tolist()):
            pa.check(self.kv.create(s, int(P)))
            slots.append(self.kv.slots(s, 0, int(P)))
        slots = np.concatenate(slots).astype(np.int32)
        self.kv.write(to_device_raw(w.k_tok, w.kv_dtype, DEV),
                      to_device_raw(w.v_tok, w.kv_dtype, DEV), torch.from_numpy(slots).to(DEV))
        offs = w.token_offsets()
        self.rows = np.concatenate([np.arange(offs[s] + a, offs[s] + a + n)
                                    for s, a, n in w.slices]).astype(np.int64)
        self.q = to_device_raw(w.q_tok[self.rows], w.q_dtype, DEV)
        q_lens = [n for _, _, n in w.slices]
        self.cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        self.seq_lens = np.array([a + n for _, a, n in w.slices], dtype=np.int32)
        seqs = [s for s, _, _ in w.slices]
        self.max_blocks = max(1, max(-(-int(P) // 16) for P in w.prompts))
        tables, _ = self.kv.pack(seqs, self.max_blocks)
        self.tables = torch.from_numpy(tables).to(DEV)
        self.d_cu = torch.from_numpy(self.cu).to(DEV)
        self.d_lens = torch.from_numpy(self.seq_lens).to(DEV)
        pf = w.slices[n_dec:]
        self.max_q = max([n for _, _, n in pf], default=0)
        self.max_dec = int(self.seq_lens[:n_dec].max()) if n_dec else 0
        self.max_pf = int(self.seq_lens[n_dec:].max()) if len(pf) else 0

    def fused(self, bufs=None, max_q=None, max_dec=None, max_pf=None):
        w = self.w
        max_q = self.max_q if max_q is None else max_q
        max_dec = self.max_dec if max_dec is None else max_dec
        max_pf = self.max_pf if max_pf is None else max_pf
        if bufs is None:
            bufs = varlen_buffers(self.n_dec, len(w.slices) - self.n_dec, w.h_q, w.h_kv, w.d,
                                  max_q, max_dec, max_pf, DEV)
        out = filled((len(self.rows), w.h_q, w.d), torch.bfloat16, DEV)
        nd = self.n_dec
        self.kv.attend_varlen(out, self.q, self.d_cu, self.d_lens, nd, self.tables[:nd],
                              self.tables[nd:], max_q, max_dec, max_pf, w.sm_scale, bufs)
        torch.cuda.synchronize()
        return to_host_raw(out, w.q_dtype), bufs

    def separate(self):
        """pa_decode over the decode rows and pa_prefill_chunk over the
        slices, into one output."""
        w, nd = self.w, self.n_dec
        out = filled((len(self.rows), w.h_q, w.d), torch.bfloat16, DEV)
        if nd:
            ws = decode_workspace(nd, w.h_q, w.h_kv, w.d, self.max_dec, DEV)
            self.kv.decode(out[:nd], self.q[:nd], self.tables[:nd].contiguous(),
                           self.d_lens[:nd].contiguous(), self.max_dec, w.sm_scale, ws)
        n_pf = len(w.slices) - nd
        if n_pf:
            cu = torch.from_numpy((self.cu[nd:] - self.cu[nd]).astype(np.int32)).to(DEV)
            q_lens = self.cu[nd + 1:] - self.cu[nd:-1]
            start = torch.from_numpy((self.seq_lens[nd:] - q_lens).astype(np.int32)).to(DEV)
            ws = prefill_workspace(n_pf, max(1, self.max_q), w.h_q, w.h_kv, w.d, self.max_pf, DEV)
            r0 = int(self.cu[nd])
            self.kv.prefill(out[r0:], self.q[r0:], cu, start, self.tables[nd:].contiguous(),
                            self.max_q, self.max_pf, w.sm_scale, ws)
        torch.cuda.synchronize()
        return to_host_raw(out, w.q_dtype)




def oracle_varlen(w):
    """The oracle's output for every row of the batch (decode rows as
    one-query slices at their last position)."""
    return oracle_prefill_run(w)["out"]
