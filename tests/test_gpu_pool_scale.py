"""GPU parity at the scale of the continuous-batching trace's pool.

ARTICLE 2.2 pre-allocates the whole block pool; at 0.9 of 288 GB and 64 KiB
per block (16 tokens x K and V x 8 KV heads x 128 dims x bf16) that is
3,955,078 blocks.  Past block id 131,072 a block's first element lies beyond
2^31 elements of its pool, so every kernel must address the cache with
64-bit offsets.  The FIFO trace only ever reaches low ids, hence:

* a pool of 140,000 blocks whose free order hands out the top ids first, the
  caches filled with NaN bit patterns (nothing unwritten may leak into an
  output), cache write + decode + a prefill slice against the oracle;
* the trace itself at its real shape (64 query / 8 KV heads, head dim 128,
  the literal pool size for the scheduler), every iteration's batch checked
  against the oracle's scheduler and three sampled iterations' attention
  against the oracle's scatter and fp64 attention."""
import collections
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_host_amd._pa as pa
import workloads
from oracle import allocator as oa
from oracle import attention as oat
from oracle import cache as oc
from oracle import codecs
from oracle.scheduler import Scheduler
from paged_kv_cache_host_amd.engine import (PagedKV, decode_workspace, prefill_workspace,
                                            sm_scale_for, to_device_raw, to_host_raw)
from tests.parity import SENTINEL, assert_close, filled, out_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
H_Q, H_KV, D = 64, 8, 128


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_pool_past_2_31_elements():
    nb = 140_000
    assert (nb - 8_000) * H_KV * D * 16 > 2 ** 31
    rng = np.random.default_rng(4400)
    top = np.arange(nb - 4000, nb, dtype=np.int32)
    order = np.concatenate([rng.permutation(top), np.arange(nb - 4000, dtype=np.int32)])
    lengths = [1, 17, 2049, 5000, 300, 16, 4097, 777]
    S = len(lengths)
    say(f"[pool scale] {nb} blocks ({2 * nb * H_KV * D * 16 * 2 / 1e9:.1f} GB), lengths {lengths}")
    kv = PagedKV(nb, H_KV, D, "bf16", DEV, order)
    kv.k.view(torch.int16).fill_(-1)     # bf16 0xFFFF: NaN
    kv.v.view(torch.int16).fill_(-1)
    opool = oa.BlockPool(nb, 16, order.tolist())
    slots = []
    for s, L in enumerate(lengths):
        assert kv.create(s, L) == pa.PA_OK and opool.seq_create(s, L) == oa.OK
        sl = kv.slots(s, 0, L)
        assert list(sl) == opool.slots(s, 0, L)
        slots.append(np.asarray(sl, dtype=np.int64))
    slots = np.concatenate(slots)
    assert slots.min() // 16 >= nb - 4000, "the sequences hold the top block ids"
    ntok = len(slots)
    k_raw = workloads.normal_raw(rng, (ntok, H_KV, D), "bf16")
    v_raw = workloads.normal_raw(rng, (ntok, H_KV, D), "bf16")
    kv.write(to_device_raw(k_raw, "bf16", DEV), to_device_raw(v_raw, "bf16", DEV),
             torch.from_numpy(slots.astype(np.int32)).to(DEV))
    # the written cells, read back from the device, against the oracle's
    # scatter into a compact pool holding just the used blocks
    used = np.unique(slots // 16)
    remap = {int(b): i for i, b in enumerate(used)}
    ckc, cvc = oc.new_cache(len(used), H_KV, 16, D, "bf16")
    cslots = np.array([remap[int(s) // 16] * 16 + int(s) % 16 for s in slots])
    oc.cache_write(ckc, cvc, k_raw, v_raw, cslots, "bf16", "bf16")
    b_t = torch.from_numpy(slots // 16).to(DEV)
    o_t = torch.from_numpy(slots % 16).to(DEV)
    got_k = to_host_raw(kv.k[b_t, :, :, o_t, :], "bf16")
    got_v = to_host_raw(kv.v[b_t, :, :, o_t], "bf16")
    assert np.array_equal(got_k, ckc[cslots // 16, :, :, cslots % 16, :])
    assert np.array_equal(got_v, cvc[cslots // 16, :, :, cslots % 16])
    # decode of every sequence
    sm = sm_scale_for(D)
    tables, lens = kv.pack(list(range(S)))
    for s in range(S):
        assert tables[s][:len(opool.block_table(s))].tolist() == opool.block_table(s)
    ctables = np.array([[remap[int(b)] if b >= 0 else -1 for b in row] for row in tables])
    q = workloads.normal_raw(rng, (S, H_Q, D), "bf16")
    out = filled((S, H_Q, D), torch.bfloat16, DEV)
    mc = int(max(lengths))
    kv.decode(out, to_device_raw(q, "bf16", DEV), torch.from_numpy(tables).to(DEV),
              torch.from_numpy(lens).to(DEV), mc, sm, decode_workspace(S, H_Q, H_KV, D, mc, DEV))
    torch.cuda.synchronize()
    ref = oat.decode(codecs.decode(q, "bf16"), ckc, cvc, ctables, lens, H_KV, sm, "bf16")
    err = assert_close(out_to_f64(to_host_raw(out, "bf16"), "bf16"), ref, "bf16", "pool-scale decode")
    say(f"    decode max|d| = {err:.3g}")
    # the last 300 positions of the 5000-token sequence as one prefill slice
    s, a, n = 3, 4700, 300
    qp = workloads.normal_raw(rng, (n, H_Q, D), "bf16")
    outp = filled((n, H_Q, D), torch.bfloat16, DEV)
    kv.prefill(outp, to_device_raw(qp, "bf16", DEV), torch.tensor([0, n], dtype=torch.int32,
                                                                  device=DEV),
               torch.tensor([a], dtype=torch.int32, device=DEV),
               torch.from_numpy(tables[s:s + 1].copy()).to(DEV), n, a + n, sm,
               prefill_workspace(1, n, H_Q, H_KV, D, a + n, DEV))
    torch.cuda.synchronize()
    refp = oat.prefill_chunk(codecs.decode(qp, "bf16"), a, ckc, cvc, ctables[s], H_KV, sm, "bf16")
    err = assert_close(out_to_f64(to_host_raw(outp, "bf16"), "bf16"), refp, "bf16",
                       "pool-scale prefill")
    say(f"    prefill max|d| = {err:.3g}")
    kv.close()


class _Tokens:
    """Per-position K/V/Q of the trace's sequences, drawn in 64-row chunks
    (workloads.seq_token_chunk) and kept in a bounded cache."""

    ROWS = 64

    def __init__(self, seed, cap=768):
        self.seed, self.cap = seed, cap
        self.chunks = collections.OrderedDict()

    def _chunk(self, sid, c):
        key = (sid, c)
        if key in self.chunks:
            self.chunks.move_to_end(key)
            return self.chunks[key]
        val = workloads.seq_token_chunk(self.seed, sid, c, self.ROWS, H_Q, H_KV, D)
        self.chunks[key] = val
        if len(self.chunks) > self.cap:
            self.chunks.popitem(last=False)
        return val

    def rows(self, seqs, positions):
        k = np.empty((len(seqs), H_KV, D), np.uint16)
        v = np.empty((len(seqs), H_KV, D), np.uint16)
        q = np.empty((len(seqs), H_Q, D), np.uint16)
        for i, (s, p) in enumerate(zip(seqs, positions)):
            ck, cv, cq = self._chunk(int(s), int(p) // self.ROWS)
            r = int(p) % self.ROWS
            k[i], v[i], q[i] = ck[r], cv[r], cq[r]
        return k, v, q


def test_trace_real_shape_sampled_iterations():
    from paged_kv_cache_host_amd.iteration import LayerIterations

    ITERS, SAMPLES, SEED = 240, (80, 160, 239), 5
    w = workloads.trace(seed=SEED, iters=ITERS)
    R, B = 256, 512
    max_ctx = max(p + o for row in w.arrivals for _, p, o in row)
    # host-only dry run of the library's scheduler: the highest block id the
    # first ITERS iterations reach sizes the device cache
    st, pool = pa.pa_pool_create(w.num_blocks, 16, None)
    assert st == pa.PA_OK
    st, sch_c = pa.pa_sched_create(pool, R, B, 16)
    assert st == pa.PA_OK
    b = pa.SchedBatch(R, B)
    top = 0
    for it in range(ITERS):
        for sid, p, o in w.arrivals[it]:
            assert pa.pa_sched_add(sch_c, sid, p, o) == pa.PA_OK
        assert pa.pa_sched_step(sch_c, b) == pa.PA_OK
        if b.n_decode:
            top = max(top, int(b.decode()[2].max()) // 16)
        if b.n_prefill_tokens:
            top = max(top, int(b.slots().max()) // 16)
    pa.pa_sched_destroy(sch_c)
    pa.pa_pool_destroy(pool)
    cache_blocks = top + 1
    say(f"[trace real shape] {ITERS} iterations, pool {w.num_blocks} blocks, device cache "
        f"{cache_blocks} blocks, samples {SAMPLES}")
    tokens = _Tokens(SEED)

    def provider(seqs, positions):
        k, v, q = tokens.rows(seqs, positions)
        return (to_device_raw(k, "bf16", DEV), to_device_raw(v, "bf16", DEV),
                to_device_raw(q, "bf16", DEV))

    run = LayerIterations(w.num_blocks, H_Q, H_KV, D, DEV, provider, R, B, max_context=max_ctx,
                          cache_blocks=cache_blocks, fill_outputs=SENTINEL)
    opool = oa.BlockPool(w.num_blocks, 16)
    sch = Scheduler(opool, R, B)
    kc, vc = oc.new_cache(cache_blocks, H_KV, 16, D, "bf16")
    sm = run.sm
    checked = {"decode": 0, "prefill": 0}
    for it in range(ITERS):
        for sid, p, o in w.arrivals[it]:
            run.add(sid, p, o)
            sch.add(sid, p, o)
        kept = []
        run.step((lambda rec, od, op: kept.append((rec, od, op))) if it in SAMPLES else None)
        rec = run.outputs()[0]
        ob = sch.step()
        ds, dp = rec["decode"]
        ps, pst, pl = rec["prefill"]
        assert [(s, p) for s, p, _ in ob.decode] == list(zip(ds.tolist(), dp.tolist())), it
        assert [(s, a, n) for s, a, n, _ in ob.prefill] == \
            list(zip(ps.tolist(), pst.tolist(), pl.tolist())), it
        for s, a, n, slots in ob.prefill:
            k, v, _ = tokens.rows([s] * n, range(a, a + n))
            oc.cache_write(kc, vc, k, v, slots, "bf16", "bf16")
        if ob.decode:
            k, v, _ = tokens.rows([s for s, _, _ in ob.decode], [p for _, p, _ in ob.decode])
            oc.cache_write(kc, vc, k, v, [sl for _, _, sl in ob.decode], "bf16", "bf16")
        if it not in SAMPLES:
            continue
        _, od, op = kept[0]
        off = 0
        worst = 0.0
        for s, a, n, _ in ob.prefill:
            _, _, q = tokens.rows([s] * n, range(a, a + n))
            ref = oat.prefill_chunk(codecs.decode(q, "bf16"), a, kc, vc, opool.block_table(s),
                                    H_KV, sm, "bf16")
            got = out_to_f64(to_host_raw(op[off:off + n], "bf16"), "bf16")
            worst = max(worst, assert_close(got, ref, "bf16", f"iteration {it} prefill seq {s}"))
            off += n
            checked["prefill"] += n
        if ob.decode:
            seqs = [s for s, _, _ in ob.decode]
            _, _, q = tokens.rows(seqs, [p for _, p, _ in ob.decode])
            mb = max(len(opool.block_table(s)) for s in seqs)
            tables = np.full((len(seqs), mb), -1, np.int64)
            for i, s in enumerate(seqs):
                t = opool.block_table(s)
                tables[i, :len(t)] = t
            lens = np.array([p + 1 for _, p, _ in ob.decode])
            ref = oat.decode(codecs.decode(q, "bf16"), kc, vc, tables, lens, H_KV, sm, "bf16")
            got = out_to_f64(to_host_raw(od, "bf16"), "bf16")
            worst = max(worst, assert_close(got, ref, "bf16", f"iteration {it} decode"))
            checked["decode"] += len(seqs)
        say(f"    iteration {it}: {len(ob.decode)} decodes, "
            f"{sum(n for _, _, n, _ in ob.prefill)} prefill tokens, max|d| = {worst:.3g}")
    run.close()
    assert checked["decode"] > 20 and checked["prefill"] > 100, checked
