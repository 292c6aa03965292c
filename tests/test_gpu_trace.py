"""GPU parity of whole continuous-batching iterations: libpa's scheduler,
cache write, decode and prefill kernels (LayerIterations) against the
oracle's scheduler, cache scatter and fp64 attention, every iteration of a
small trace whose pool is tight enough to preempt."""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import allocator as oa
from oracle import attention as oat
from oracle import cache as oc
from oracle import codecs
from oracle.scheduler import Scheduler
from tests.parity import assert_close

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_trace_iterations_match_oracle():
    from paged_kv_cache_host_amd.engine import to_device_raw
    from paged_kv_cache_host_amd.iteration import LayerIterations

    H_Q, H_KV, D, R, B, SEED = 16, 4, 128, 12, 96, 41
    w = workloads.trace(seed=SEED, iters=80, lam=0.5, prompt_median=60, prompt_sigma=0.8,
                        prompt_cap=500, out_mean=30, num_blocks=80)
    say(f"[trace parity] {w.name} pool={w.num_blocks} running<={R} budget={B}")
    rows = {}
    for row in w.arrivals:
        for sid, p, o in row:
            rows[sid] = workloads.seq_token_rows(SEED, sid, p + o, H_Q, H_KV, D)

    def host_rows(seqs, positions):
        k = np.stack([rows[s][0][p] for s, p in zip(seqs, positions)])
        v = np.stack([rows[s][1][p] for s, p in zip(seqs, positions)])
        q = np.stack([rows[s][2][p] for s, p in zip(seqs, positions)])
        return k, v, q

    def provider(seqs, positions):
        k, v, q = host_rows(seqs, positions)
        return (to_device_raw(k, "bf16", "cuda"), to_device_raw(v, "bf16", "cuda"),
                to_device_raw(q, "bf16", "cuda"))

    max_ctx = max(p + o for row in w.arrivals for _, p, o in row)
    run = LayerIterations(w.num_blocks, H_Q, H_KV, D, "cuda", provider, R, B, max_context=max_ctx)
    pool = oa.BlockPool(w.num_blocks, 16)
    sch = Scheduler(pool, R, B)
    kc, vc = oc.new_cache(w.num_blocks, H_KV, 16, D, "bf16")
    sm = run.sm
    checked = {"decode": 0, "prefill": 0}
    worst = [0.0]

    for it in range(w.iters):
        for sid, p, o in w.arrivals[it]:
            run.add(sid, p, o)
            sch.add(sid, p, o)
        got = {}

        def keep(rec, out_dec, out_pf):
            got["rec"] = rec
            got["dec"] = codecs.decode(out_dec.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
            got["pf"] = codecs.decode(out_pf.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")

        run.step(keep)
        ob = sch.step()
        ds, dp = got["rec"]["decode"]
        ps, pst, pl = got["rec"]["prefill"]
        assert [(s, p) for s, p, _ in ob.decode] == list(zip(ds.tolist(), dp.tolist())), it
        assert [(s, a, n) for s, a, n, _ in ob.prefill] == \
            list(zip(ps.tolist(), pst.tolist(), pl.tolist())), it
        # oracle: write this iteration's tokens, then attend
        for s, a, n, slots in ob.prefill:
            k, v, _ = host_rows([s] * n, list(range(a, a + n)))
            oc.cache_write(kc, vc, k, v, slots, "bf16", "bf16")
        for s, p, slot in ob.decode:
            k, v, _ = host_rows([s], [p])
            oc.cache_write(kc, vc, k, v, [slot], "bf16", "bf16")
        off = 0
        for s, a, n, _ in ob.prefill:
            _, _, q = host_rows([s] * n, list(range(a, a + n)))
            ref = oat.prefill_chunk(codecs.decode(q, "bf16"), a, kc, vc, pool.block_table(s),
                                    H_KV, sm, "bf16")
            worst[0] = max(worst[0], assert_close(got["pf"][off:off + n], ref, "bf16",
                                                  f"iteration {it} prefill seq {s}"))
            off += n
            checked["prefill"] += n
        if ob.decode:
            seqs = [s for s, _, _ in ob.decode]
            _, _, q = host_rows(seqs, [p for _, p, _ in ob.decode])
            mb = max(len(pool.block_table(s)) for s in seqs)
            tables = np.full((len(seqs), mb), -1, np.int64)
            for i, s in enumerate(seqs):
                t = pool.block_table(s)
                tables[i, :len(t)] = t
            lens = np.array([p + 1 for _, p, _ in ob.decode])
            ref = oat.decode(codecs.decode(q, "bf16"), kc, vc, tables, lens, H_KV, sm, "bf16")
            worst[0] = max(worst[0], assert_close(got["dec"], ref, "bf16", f"iteration {it} decode"))
            checked["decode"] += len(seqs)
    run.close()
    say(f"    checked {checked['decode']} decode tokens, {checked['prefill']} prefill tokens, "
        f"{run.totals['preempted']} preemptions, max|d| = {worst[0]:.3g}")
    assert run.totals["preempted"] > 0 and checked["decode"] > 50 and checked["prefill"] > 500
