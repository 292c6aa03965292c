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
from tests.parity import SENTINEL, assert_close

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


H_Q, H_KV, D, R, B, SEED = 16, 4, 128, 12, 96, 41


# prefill budget per schedule (static: members x longest prompt)
BUDGET = {"chunked": B, "continuous": 256, "static": R * 500, "naive": 256}


def _trace():
    w = workloads.trace(seed=SEED, iters=80, lam=0.5, prompt_median=60, prompt_sigma=0.8,
                        prompt_cap=500, out_mean=30, num_blocks=80)
    # rows for every position a request can reach, padding of a static batch
    # included (at most the longest prompt plus the longest output)
    n_rows = max(p for row in w.arrivals for _, p, _ in row) + \
        max(o for row in w.arrivals for _, _, o in row)
    rows = {}
    for row in w.arrivals:
        for sid, p, o in row:
            rows[sid] = workloads.seq_token_rows(SEED, sid, n_rows, H_Q, H_KV, D)

    def host_rows(seqs, positions):
        k = np.stack([rows[s][0][p] for s, p in zip(seqs, positions)])
        v = np.stack([rows[s][1][p] for s, p in zip(seqs, positions)])
        q = np.stack([rows[s][2][p] for s, p in zip(seqs, positions)])
        return k, v, q

    return w, host_rows, n_rows


def _replay(w, host_rows, sm, results, mode="chunked", ids=None, retain=False, cache="bf16",
            scale=1.0):
    """Run the oracle's scheduler, cache scatter and attention over the same
    trace and compare every iteration's record and outputs (``results[it]``
    = (record, decode output, prefill output), decoded to float).  ``ids``:
    prompt token ids per request (prefix caching)."""
    pool = oa.BlockPool(w.num_blocks, 16)
    pool.set_prefix_retention(retain)
    sch = Scheduler(pool, R, BUDGET[mode], mode=mode)
    kc, vc = oc.new_cache(w.num_blocks, H_KV, 16, D, cache)
    checked = {"decode": 0, "prefill": 0}
    worst = 0.0
    written = set()
    for it in range(w.iters):
        for sid, p, o in w.arrivals[it]:
            if ids is not None:
                sch.add_prompt(sid, p, o, ids[sid])
            else:
                sch.add(sid, p, o)
        rec, dec, pf = results[it]
        ob = sch.step()
        ds, dp = rec["decode"]
        ps, pst, pl = rec["prefill"]
        assert [(s, p) for s, p, _ in ob.decode] == list(zip(ds.tolist(), dp.tolist())), it
        assert [(s, a, n) for s, a, n, _ in ob.prefill] == \
            list(zip(ps.tolist(), pst.tolist(), pl.tolist())), it
        # oracle: write this iteration's tokens, then attend
        for s, a, n, slots in ob.prefill:
            k, v, _ = host_rows([s] * n, list(range(a, a + n)))
            oc.cache_write(kc, vc, k, v, slots, "bf16", cache, scale, scale)
            written.update(int(x) for x in slots)
        for s, p, slot in ob.decode:
            k, v, _ = host_rows([s], [p])
            oc.cache_write(kc, vc, k, v, [slot], "bf16", cache, scale, scale)
            written.add(int(slot))
        off = 0
        for s, a, n, _ in ob.prefill:
            _, _, q = host_rows([s] * n, list(range(a, a + n)))
            ref = oat.prefill_chunk(codecs.decode(q, "bf16"), a, kc, vc, pool.block_table(s),
                                    H_KV, sm, cache, scale, scale)
            worst = max(worst, assert_close(pf[off:off + n], ref, cache,
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
            ref = oat.decode(codecs.decode(q, "bf16"), kc, vc, tables, lens, H_KV, sm, cache,
                             scale, scale)
            worst = max(worst, assert_close(dec, ref, cache, f"iteration {it} decode"))
            checked["decode"] += len(seqs)
    if ids is not None:
        checked["prefix_hits"] = sch.prefix_hits
    return checked, worst, kc, vc, sorted(written)


def _decode_bf16(t):
    return codecs.decode(t.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")


@pytest.mark.parametrize("mode,fused", [("chunked", False), ("continuous", False),
                                        ("static", False), ("naive", False), ("chunked", True),
                                        ("static", True)])
def test_trace_iterations_match_oracle(mode, fused):
    """Host waits for every iteration's kernels (the ``keep`` callback); each
    of the four schedules (static batches prefill up to 12 padded prompts in
    one launch); ``fused``: each iteration's attention is one
    pa_attend_varlen launch over its decode rows and slices."""
    from paged_kv_cache_host_amd.engine import to_device_raw
    from paged_kv_cache_host_amd.iteration import LayerIterations

    w, host_rows, max_ctx = _trace()
    say(f"[trace parity, synchronous, {mode}, fused={fused}] {w.name} pool={w.num_blocks} "
        f"running<={R} budget={BUDGET[mode]}")

    def provider(seqs, positions):
        k, v, q = host_rows(seqs, positions)
        return (to_device_raw(k, "bf16", "cuda"), to_device_raw(v, "bf16", "cuda"),
                to_device_raw(q, "bf16", "cuda"))

    run = LayerIterations(w.num_blocks, H_Q, H_KV, D, "cuda", provider, R, BUDGET[mode],
                          max_context=max_ctx, mode=mode, fill_outputs=SENTINEL, fused=fused)
    results = []
    for it in range(w.iters):
        for sid, p, o in w.arrivals[it]:
            run.add(sid, p, o)

        def keep(rec, out_dec, out_pf):
            results.append((rec, _decode_bf16(out_dec), _decode_bf16(out_pf)))

        run.step(keep)
    run.close()
    checked, worst, _, _, _ = _replay(w, host_rows, run.sm, results, mode)
    say(f"    checked {checked['decode']} decode tokens, {checked['prefill']} prefill tokens, "
        f"{run.totals['preempted']} preemptions, max|d| = {worst:.3g}")
    assert checked["decode"] > 50 and checked["prefill"] > 500
    if mode == "chunked":
        assert run.totals["preempted"] > 0


@pytest.mark.parametrize("two_streams,fused", [(False, False), (True, False), (False, True)])
def test_trace_iterations_pipelined_match_oracle(two_streams, fused):
    """The host runs ahead of the kernels (metadata ring, one event per group
    of iterations, provider tensors already resident): outputs are copied on
    the compute stream, the written cache slots compared byte for byte at
    the end."""
    from paged_kv_cache_host_amd.engine import to_device_raw
    from paged_kv_cache_host_amd.iteration import LayerIterations

    w, host_rows, max_ctx = _trace()
    say(f"[trace parity, pipelined, two_streams={two_streams}, fused={fused}] {w.name} "
        f"pool={w.num_blocks} running<={R} budget={B}")

    def provider(seqs, positions):
        k, v, q = host_rows(seqs, positions)
        out = (to_device_raw(k, "bf16", "cuda"), to_device_raw(v, "bf16", "cuda"),
               to_device_raw(q, "bf16", "cuda"))
        torch.cuda.current_stream().synchronize()
        return out

    run = LayerIterations(w.num_blocks, H_Q, H_KV, D, "cuda", provider, R, B, max_context=max_ctx,
                          provider_syncs=False, two_streams=two_streams, fill_outputs=SENTINEL,
                          fused=fused)
    copies = []
    for it in range(w.iters):
        for sid, p, o in w.arrivals[it]:
            run.add(sid, p, o)
        run.step()
        rec, od, op = run.outputs()
        with torch.cuda.stream(run.compute):
            copies.append((rec, od.clone(), op.clone()))
    run.synchronize()
    results = [(rec, _decode_bf16(od), _decode_bf16(op)) for rec, od, op in copies]
    k_dev = run.k.view(torch.int16).cpu().numpy().view(np.uint16)
    v_dev = run.v.view(torch.int16).cpu().numpy().view(np.uint16)
    run.close()
    checked, worst, kc, vc, written = _replay(w, host_rows, run.sm, results)
    blk = np.array(written) // 16
    off = np.array(written) % 16
    np.testing.assert_array_equal(k_dev[blk, :, :, off, :], kc[blk, :, :, off, :])
    np.testing.assert_array_equal(v_dev[blk, :, :, off], vc[blk, :, :, off])
    say(f"    checked {checked['decode']} decode tokens, {checked['prefill']} prefill tokens, "
        f"{len(written)} cache slots, {run.totals['preempted']} preemptions, max|d| = {worst:.3g}")
    assert run.totals["preempted"] > 0 and checked["decode"] > 50 and checked["prefill"] > 500


@pytest.mark.parametrize("mode", ["chunked", "continuous", "static", "naive"])
def test_serve_live_clock(mode):
    """``serve`` on a live clock: every request is released with exactly its
    target count of output tokens, one inter-token gap per token after the
    first, a positive time to first token (no token before its arrival),
    and every request within targets no schedule can miss."""
    from paged_kv_cache_host_amd.iteration import LayerIterations, serve

    reqs = workloads.timed_requests(seed=21, n=24, rate_per_ms=20.0, prompt_median=40,
                                    prompt_cap=300, out_mean=6, out_cap=40)
    say(f"[serve, {mode}] {len(reqs)} requests, budget {BUDGET[mode]}")
    ring = 2 * (R + BUDGET[mode])
    g = torch.Generator(device="cuda")
    g.manual_seed(22)
    kr = torch.randn((ring, H_KV, D), generator=g, device="cuda").to(torch.bfloat16)
    vr = torch.randn((ring, H_KV, D), generator=g, device="cuda").to(torch.bfloat16)
    qr = torch.randn((ring, H_Q, D), generator=g, device="cuda").to(torch.bfloat16)

    def provider(seqs, positions):
        n = len(seqs)
        return kr[:n], vr[:n], qr[:n]

    max_ctx = max(r[2] for r in reqs) + max(r[3] for r in reqs)
    run = LayerIterations(400, H_Q, H_KV, D, "cuda", provider, R, BUDGET[mode],
                          max_context=max_ctx, provider_syncs=False, mode=mode)
    r = serve(run, reqs, ttft_slo_ms=1e9, itl_slo_ms=1e9, timeout_s=60.0)
    run.close()
    assert run.totals["finished"] == len(reqs)
    assert r["output_tokens"] == sum(x[3] for x in reqs)
    assert r["slo_met_requests"] == len(reqs)        # targets no request can miss
    assert r["ttft"]["n"] == len(reqs) and r["ttft"]["min_ms"] > 0
    assert r["itl"]["n"] == sum(x[3] - 1 for x in reqs)
    assert r["itl"]["max_ms"] >= 0 and r["iterations"] > max(x[3] for x in reqs)
    say(f"    {r['iterations']} iterations, {r['wall_s'] * 1e3:.2f} ms, "
        f"TTFT mean {r['ttft']['mean_ms']:.3f} ms")


def _prefix_trace(lam=0.5, iters=80, out_mean=30):
    """The trace above with every prompt behind one of three system prefixes
    (40, 64 and 100 tokens) and its own tokens after it.  A prefix's token
    rows are the same for every request that starts with it, as its K/V
    would be; prompt token ids are the prefix's ids, then the request's."""
    from types import SimpleNamespace
    base = workloads.trace(seed=SEED + 1, iters=iters, lam=lam, prompt_median=40,
                           prompt_sigma=0.8, prompt_cap=300, out_mean=out_mean, num_blocks=80)
    rng = np.random.default_rng(SEED)
    plens = [40, 64, 100]
    pids = [rng.integers(0, 30000, n).astype(np.int32) for n in plens]
    arrivals, ids, src = [], {}, {}
    for row in base.arrivals:
        out = []
        for sid, p, o in row:
            k = int(rng.integers(0, 3))
            ids[sid] = np.concatenate([pids[k], rng.integers(30000, 60000, p).astype(np.int32)])
            src[sid] = (k, plens[k])
            out.append((sid, plens[k] + p, o))
        arrivals.append(out)
    w = SimpleNamespace(arrivals=arrivals, iters=base.iters, num_blocks=base.num_blocks,
                        name=base.name + " behind 3 shared prefixes")
    n_rows = max(p for row in arrivals for _, p, _ in row) + \
        max(o for row in arrivals for _, _, o in row)
    prefix_rows = [workloads.seq_token_rows(SEED, 100000 + k, n, H_Q, H_KV, D)
                   for k, n in enumerate(plens)]
    rows = {sid: workloads.seq_token_rows(SEED, sid, n_rows, H_Q, H_KV, D)
            for row in arrivals for sid, _, _ in row}

    def row_of(s, p):
        k, n = src[s]
        return (prefix_rows[k], p) if p < n else (rows[s], p)

    def host_rows(seqs, positions):
        got = [row_of(s, p) for s, p in zip(seqs, positions)]
        return tuple(np.stack([r[j][p] for r, p in got]) for j in range(3))

    return w, host_rows, n_rows, ids


@pytest.mark.parametrize("retain,lam,iters,out_mean,min_hits,cache",
                         [(False, 0.5, 80, 30, 200, "bf16"), (True, 0.1, 160, 10, 500, "bf16"),
                          (False, 0.5, 80, 30, 200, "fp8")])
def test_trace_prefix_caching_matches_oracle(retain, lam, iters, out_mean, min_hits, cache):
    """Prefix caching through whole iterations: requests queued with their
    prompt token ids share the prompt blocks earlier requests computed, and
    prefill only after them; with ``retain`` (sparser arrivals) the pool
    keeps finished requests' prompt blocks findable, so later requests also
    attend blocks brought back from retention.  Schedule, cache and every
    decode and prefill output against the oracle's scheduler (same
    readings) and fp64 attention over the same cache."""
    from paged_kv_cache_host_amd import _pa as pa
    from paged_kv_cache_host_amd.engine import to_device_raw
    from paged_kv_cache_host_amd.iteration import LayerIterations

    w, host_rows, max_ctx, ids = _prefix_trace(lam, iters, out_mean)
    scale = (4.9 / 448.0) if cache == "fp8" else 1.0   # e4m3 scale of N(0,1) rows
    say(f"[trace parity, prefix caching, retain={retain}, {cache}] {w.name} "
        f"pool={w.num_blocks} running<={R} budget={B}")

    def provider(seqs, positions):
        k, v, q = host_rows(seqs, positions)
        return (to_device_raw(k, "bf16", "cuda"), to_device_raw(v, "bf16", "cuda"),
                to_device_raw(q, "bf16", "cuda"))

    run = LayerIterations(w.num_blocks, H_Q, H_KV, D, "cuda", provider, R, B,
                          max_context=max_ctx, fill_outputs=SENTINEL, cache_dtype=cache,
                          k_scale=scale, v_scale=scale)
    pa.check(pa.pa_pool_set_prefix_retention(run.pool, retain))
    results = []
    for it in range(w.iters):
        for sid, p, o in w.arrivals[it]:
            run.add(sid, p, o, ids=ids[sid])

        def keep(rec, out_dec, out_pf):
            results.append((rec, _decode_bf16(out_dec), _decode_bf16(out_pf)))

        run.step(keep)
    hits = run.acc["prefix_hit_tokens"]
    run.close()
    checked, worst, _, _, _ = _replay(w, host_rows, run.sm, results, ids=ids, retain=retain,
                                      cache=cache, scale=scale)
    say(f"    checked {checked['decode']} decode tokens, {checked['prefill']} prefill tokens, "
        f"{hits} prompt tokens found shared, {run.totals['preempted']} preemptions, "
        f"max|d| = {worst:.3g}")
    # (with retention the sparse trace finds 768 prompt tokens, 160 without)
    assert hits == checked["prefix_hits"] and hits > min_hits
    assert checked["decode"] > 50 and checked["prefill"] > 300
