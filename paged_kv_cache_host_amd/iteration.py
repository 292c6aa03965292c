"""One attention layer driven through continuous-batching iterations.

Each ``step`` is one iteration of the LESSON's loop ("Continuous batching at
the iteration level", "Chunked prefill"): libpa's scheduler (pa_sched_step)
grows the decode-phase sequences by one token, admits and hands out prefill
slices within the budget; the new tokens' K/V are scattered into the paged
cache (pa_cache_write) and attention runs for the decode tokens (pa_decode)
and the prefill slices (pa_prefill_chunk), on one compute stream (or, with
``two_streams``, the prefill beside the decode on a second stream that the
compute stream waits for at the end of the iteration).  The
host work of iteration t+1 (scheduling and table packing into a ring of
pinned buffers) overlaps the kernels of the iterations before it; one
pa_stage_cache_write launch on the compute stream then moves the packed
metadata and scatters the new tokens' K/V.

Token data (new K, V, Q rows) comes from a caller-supplied provider:
``provider(seqs, positions) -> (k [n, H_kv, D], v [n, H_kv, D], q [n, H_q, D])``
device tensors, so that a benchmark can feed a pre-generated ring and a test
can feed per-position data the oracle also sees.

Argument marshalling and buffer management only: every scheduling decision
is made in libpa's C++ scheduler and every byte of attention in its kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _pa as pa
from .engine import BLOCK, _TORCH_STORAGE, varlen_buffers


class LayerIterations:
    def __init__(self, num_blocks: int, h_q: int, h_kv: int, d: int, device, provider,
                 max_running: int = 256, prefill_budget: int = 512, max_context: int = 40960,
                 cache_blocks: int | None = None, cache_dtype: str = "bf16",
                 k_scale: float = 1.0, v_scale: float = 1.0, sm_scale: float | None = None,
                 free_order=None, provider_syncs: bool = True, two_streams: bool = False,
                 mode: str = "chunked", fill_outputs: float | None = None, fused: bool = False):
        self.h_q, self.h_kv, self.d = h_q, h_kv, d
        self.dev = torch.device(device)
        self.provider = provider
        # the provider's tensors come from work queued on the caller's
        # current stream (True) or are already in memory (False: no
        # cross-stream wait per iteration)
        self.provider_syncs = bool(provider_syncs)
        # test aid: each iteration's output rows are set to this value on the
        # compute stream before its kernels, so a row no kernel writes keeps it
        self.fill_outputs = fill_outputs
        self.R, self.B = max_running, prefill_budget
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.sm = sm_scale if sm_scale is not None else float(np.float32(1.0) / np.float32(np.sqrt(d)))
        st, self.pool = pa.pa_pool_create(num_blocks, BLOCK, free_order)
        pa.check(st)
        st, self.sched = pa.pa_sched_create_mode(self.pool, mode, max_running, prefill_budget,
                                                 BLOCK)
        pa.check(st)
        self.batch = pa.SchedBatch(max_running, prefill_budget)
        # Device cache: blocks [0, cache_blocks) are backed (all of the pool
        # by default).  The kernels clamp any table entry outside it.
        self.cache_blocks = num_blocks if cache_blocks is None else int(cache_blocks)
        dt = _TORCH_STORAGE[cache_dtype]
        x = 16 // torch.empty((), dtype=dt).element_size()
        self.k = torch.empty((self.cache_blocks, h_kv, d // x, BLOCK, x), dtype=dt, device=self.dev)
        self.v = torch.empty((self.cache_blocks, h_kv, d, BLOCK), dtype=dt, device=self.dev)
        self.max_ctx = max_context
        mb = -(-max_context // BLOCK)
        # A ring of NBUF pinned buffers, each with a device twin, holds the
        # iterations' slots, decode context lengths and tables, prefill
        # tables and slice metadata, packed back to back; one launch on the
        # compute stream moves the used prefix.  One event per GROUP
        # iterations tells the host which buffers the kernels have read.
        T = max_running + max(prefill_budget, 1)
        n_meta = T + 2 * max_running * mb + 4 * max_running + 1
        self.NBUF, self.GROUP = 8, 4
        self.host_buf = [torch.empty(n_meta, dtype=torch.int32, pin_memory=True)
                         for _ in range(self.NBUF)]
        self.dev_buf = [torch.empty(n_meta, dtype=torch.int32, device=self.dev)
                        for _ in range(self.NBUF)]
        out_dt = torch.bfloat16
        self.out_dec = [torch.empty((max_running, h_q, d), dtype=out_dt, device=self.dev) for _ in range(2)]
        self.out_pf = [torch.empty((max(prefill_budget, 1), h_q, d), dtype=out_dt, device=self.dev)
                       for _ in range(2)]
        n = pa.pa_decode_workspace_bytes(max_running, h_q, h_kv, d, max_context)
        self.ws_dec = torch.zeros(max(n, 1), dtype=torch.uint8, device=self.dev)
        # sized for every call with at most max_running slices of at most
        # the budget (the query bounds every smaller call)
        top = max(prefill_budget, 1)
        n = pa.pa_prefill_workspace_bytes(max_running, top, h_q, h_kv, d, max_context)
        self.ws_pf = torch.empty(max(n, 1), dtype=torch.uint8, device=self.dev)
        # fused: one pa_attend_varlen per iteration over [decode rows; slices]
        self.fused = bool(fused)
        if self.fused:
            self.out_mix = [torch.empty((T, h_q, d), dtype=out_dt, device=self.dev)
                            for _ in range(2)]
            self.bufs_mix = varlen_buffers(max_running, max_running, h_q, h_kv, d, top,
                                           max_context, max_context, self.dev)
        self.compute = torch.cuda.Stream(device=self.dev)
        # two_streams: the prefill slices run on a second stream, after the
        # staging launch and beside the decode, and the compute stream waits
        # for them before the iteration ends (two events per iteration)
        self.side = torch.cuda.Stream(device=self.dev) if two_streams else None
        self.ev_staged = torch.cuda.Event()
        self.ev_prefilled = torch.cuda.Event()
        self.ev_group = [torch.cuda.Event() for _ in range(2)]
        for e in self.ev_group:
            e.record(self.compute)
        self.it = 0
        self._last = None
        self.totals = {"decode_tokens": 0, "prefill_tokens": 0, "preempted": 0, "finished": 0}
        self.waste = []        # internal waste per iteration (nan: nothing held)
        self.unwritten = []    # reserved-unwritten share per iteration (nan: nothing held)

    def close(self):
        if self.sched is not None:
            pa.pa_sched_destroy(self.sched)
            self.sched = None
        if self.pool is not None:
            pa.pa_pool_destroy(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, seq: int, prompt_len: int, target: int, ids=None):
        """Queue a request; with its prompt's token ids (``ids``, prompt_len
        of them) the scheduler shares the leading prompt blocks an earlier
        request already computed (prefix caching, chunked schedule)."""
        if ids is None:
            pa.check(pa.pa_sched_add(self.sched, seq, prompt_len, target))
        else:
            if len(ids) != prompt_len:
                raise ValueError("one token id per prompt position")
            pa.check(pa.pa_sched_add_prompt(self.sched, seq, target, ids))

    def step(self, keep=None):
        """One iteration.  ``keep``: optional callback(record) receiving the
        iteration's host-side record (decode/prefill lists) and its output
        tensors once the kernels have finished (test use)."""
        X = self.it % self.NBUF
        g = self.it // self.GROUP
        if self.it % self.GROUP == 0:
            # recorded after group g-2, the last user of this group's buffers
            self.ev_group[g % 2].synchronize()
        O = self.it & 1    # output buffers: the stream orders their reuse
        b = self.batch
        pa.check(pa.pa_sched_step(self.sched, b))
        ds, dp, dsl = b.decode()
        ps, pst, pl = b.prefill()
        n_dec, n_pf, n_pt = b.n_decode, b.n_prefill, b.n_prefill_tokens
        fin, _, pre = b.events()
        self.totals["decode_tokens"] += n_dec
        self.totals["prefill_tokens"] += n_pt
        self.totals["preempted"] += len(pre)
        self.totals["finished"] += len(fin)
        st, acc = pa.pa_sched_stats(self.sched)
        pa.check(st)
        self.acc = acc
        held = acc["blocks_held"] * BLOCK
        self.waste.append(float("nan") if held == 0 else 1.0 - acc["tokens_held"] / held)
        self.unwritten.append(float("nan") if held == 0 else acc["unwritten"] / held)

        # token data: prefill tokens first, then decode tokens (fused: the
        # decode rows first, as pa_attend_varlen takes them)
        pf_pos = np.concatenate([np.arange(a, a + n) for a, n in zip(pst.tolist(), pl.tolist())]) \
            if n_pf else np.zeros(0, np.int64)
        pf_seq = np.repeat(ps, pl) if n_pf else np.zeros(0, np.int64)
        if self.fused:
            seqs = np.concatenate([ds, pf_seq]).astype(np.int64)
            poss = np.concatenate([dp, pf_pos]).astype(np.int64)
        else:
            seqs = np.concatenate([pf_seq, ds]).astype(np.int64)
            poss = np.concatenate([pf_pos, dp]).astype(np.int64)
        n_tok = n_pt + n_dec
        h = self.host_buf[X].numpy()
        dvb = self.dev_buf[X]
        off = 0

        def region(n):
            nonlocal off
            r = (h[off:off + n], dvb[off:off + n])
            off += n
            return r

        h_sl, d_sl = region(n_tok)
        if self.fused:
            h_sl[:n_dec] = dsl
            h_sl[n_dec:] = b.slots()
            h_vl, d_vl = region(n_dec + n_pf)       # seq_lens
            h_vl[:n_dec] = dp + 1
            h_vl[n_dec:] = pst + pl
            h_cu, d_cu = region(n_dec + n_pf + 1)   # cu_q_lens
            h_cu[:n_dec + 1] = np.arange(n_dec + 1)
            h_cu[n_dec + 1:] = n_dec + np.cumsum(pl)
        else:
            h_sl[:n_pt] = b.slots()
            h_sl[n_pt:] = dsl
        mbd = mbp = 1
        if n_dec:
            max_ctx_d = int(dp.max()) + 1
            mbd = -(-max_ctx_d // BLOCK)
            h_dl, d_dl = region(n_dec)
            h_dt, d_dt = region(n_dec * mbd)
            st, _, _ = pa.pa_pack_batch(self.pool, ds, mbd, h_dt.reshape(n_dec, mbd), h_dl)
            pa.check(st)
        if n_pf:
            # a prefilling sequence holds the blocks of all its known tokens
            held = 0
            for sq in ps.tolist():
                st, n = pa.pa_seq_length(self.pool, sq)
                pa.check(st)
                held = max(held, n)
            mbp = -(-held // BLOCK)
            h_pt, d_pt = region(n_pf * mbp)
            st, _, _ = pa.pa_pack_batch(self.pool, ps, mbp, h_pt.reshape(n_pf, mbp), None)
            pa.check(st)
            if not self.fused:
                h_pm, d_pm = region(2 * n_pf + 1)
                h_pm[0] = 0
                h_pm[1:n_pf + 1] = np.cumsum(pl)
                h_pm[n_pf + 1:] = pst
        record = {"decode": (ds.copy(), dp.copy()), "prefill": (ps.copy(), pst.copy(), pl.copy())}
        k_new = v_new = q_new = None
        if n_tok:
            k_new, v_new, q_new = self.provider(seqs, poss)
        c = self.compute
        if n_tok and self.provider_syncs:
            # the provider's tensors were produced on the caller's stream
            c.wait_stream(torch.cuda.current_stream(self.dev))
            for t in (k_new, v_new, q_new):
                t.record_stream(c)
        if n_tok:
            # the new tokens' slots lead the buffer: one launch stages it and
            # scatters their K/V
            pa.check(pa.pa_stage_cache_write(c, dvb, self.host_buf[X], 4 * off, 0, n_tok, k_new,
                                             v_new, self.k, self.v, self.cache_blocks, self.h_kv,
                                             self.d, BLOCK, self.k_scale, self.v_scale))
        else:
            pa.check(pa.pa_stage(c, dvb, self.host_buf[X], 4 * off))
        if self.fill_outputs is not None:
            with torch.cuda.stream(c):
                if self.fused:
                    self.out_mix[O][:n_tok].fill_(self.fill_outputs)
                else:
                    self.out_pf[O][:n_pt].fill_(self.fill_outputs)
                    self.out_dec[O][:n_dec].fill_(self.fill_outputs)
        if self.fused:
            if n_tok:
                counters, ws = self.bufs_mix
                pa.check(pa.pa_attend_varlen(
                    c, self.out_mix[O][:n_tok], q_new[:n_tok], d_cu, d_vl, n_dec, self.k, self.v,
                    d_dt.view(n_dec, mbd) if n_dec else None,
                    d_pt.view(n_pf, mbp) if n_pf else None, self.cache_blocks, self.h_kv,
                    int(pl.max()) if n_pf else 0, int(dp.max()) + 1 if n_dec else 0,
                    int((pst + pl).max()) if n_pf else 0, self.sm, self.k_scale, self.v_scale,
                    counters, ws))
            if self.it % self.GROUP == self.GROUP - 1:
                self.ev_group[g % 2].record(c)
            self._last = (record, self.out_mix[O][:n_dec], self.out_mix[O][n_dec:n_tok])
            if keep is not None:
                c.synchronize()
                keep(record, self.out_mix[O][:n_dec].clone(), self.out_mix[O][n_dec:n_tok].clone())
            self.it += 1
            return n_tok
        if n_pf:
            pf_stream = c
            if self.side is not None:
                self.ev_staged.record(c)
                self.side.wait_event(self.ev_staged)
                pf_stream = self.side
                if self.provider_syncs:
                    q_new.record_stream(pf_stream)
            pa.check(pa.pa_prefill_chunk(pf_stream, self.out_pf[O][:n_pt], q_new[:n_pt], d_pm[:n_pf + 1],
                                         d_pm[n_pf + 1:], self.k, self.v, d_pt.view(n_pf, mbp),
                                         self.cache_blocks, self.h_kv, int(pl.max()),
                                         int((pst + pl).max()), self.sm, self.k_scale,
                                         self.v_scale, self.ws_pf))
        if n_dec:
            pa.check(pa.pa_decode(c, self.out_dec[O][:n_dec], q_new[n_pt:n_tok], self.k, self.v,
                                  d_dt.view(n_dec, mbd), d_dl, self.cache_blocks, self.h_kv,
                                  int(dp.max()) + 1, self.sm, self.k_scale, self.v_scale,
                                  self.ws_dec))
        if n_pf and self.side is not None:
            # the iteration ends on the compute stream with both kernels done
            self.ev_prefilled.record(self.side)
            c.wait_event(self.ev_prefilled)
        if self.it % self.GROUP == self.GROUP - 1:
            self.ev_group[g % 2].record(c)
        self._last = (record, self.out_dec[O][:n_dec], self.out_pf[O][:n_pt])
        if keep is not None:
            c.synchronize()
            keep(record, self.out_dec[O][:n_dec].clone(), self.out_pf[O][:n_pt].clone())
        self.it += 1
        return n_tok

    def outputs(self):
        """The last iteration's host-side record and its decode and prefill
        outputs as device views.  The kernels that write them are queued on
        ``self.compute``, and the iteration after next overwrites them, so
        read them from work on that stream (or after ``synchronize``)."""
        return self._last

    def synchronize(self):
        self.compute.synchronize()


class LatencyLog:
    """Token times of a continuous-batching run (the LESSON's simulator
    reports mean time to first token and the P99 inter-token latency per
    schedule).  A request arrives before iteration a; an output token comes
    out of every iteration whose prefill slice completes the request's known
    tokens (its first token, or the next one after a preemption's
    recomputation) and out of every decode iteration, up to the request's
    target (a static batch's padding tokens past it are not counted).  Fed
    from the scheduler's batches (``pa_sched_step``).  Two clocks: the
    iteration clock (TTFT = f - a + 1 iterations, gaps in iterations, times a
    measured mean iteration time), or measured end times of every iteration
    with arrival times on the same clock (``timed``)."""

    def __init__(self):
        self.arrival, self.target, self.tokens = {}, {}, {}

    def add(self, it: int, seq: int, target: int | None = None):
        self.arrival[seq] = it
        self.target[seq] = target
        self.tokens[seq] = []

    def _token(self, seq: int, it: int):
        t = self.tokens[seq]
        cap = self.target[seq]
        if cap is None or len(t) < cap:
            t.append(it)

    def step(self, it: int, decode_seqs, prefill_seqs, prefill_emits):
        for s, e in zip(prefill_seqs, prefill_emits):
            if e:
                self._token(int(s), it)
        for s in decode_seqs:
            self._token(int(s), it)

    def ttft(self) -> np.ndarray:
        """TTFT in iterations of every request that got its first token."""
        return np.array([t[0] - self.arrival[s] + 1 for s, t in sorted(self.tokens.items()) if t],
                        dtype=np.int64)

    def itl(self) -> np.ndarray:
        """Inter-token gaps in iterations, all requests, in request order."""
        gaps = [np.diff(np.asarray(t, dtype=np.int64)) for _, t in sorted(self.tokens.items())]
        return np.concatenate(gaps) if gaps else np.zeros(0, np.int64)

    def summary(self, ms_per_iteration: float) -> dict:
        t, g = self.ttft(), self.itl()

        def stats(x):
            if len(x) == 0:
                return {"n": 0}
            return {"n": int(len(x)), "mean_it": float(x.mean()),
                    "p50_it": float(np.percentile(x, 50)), "p99_it": float(np.percentile(x, 99)),
                    "max_it": int(x.max()), "mean_ms": float(x.mean() * ms_per_iteration),
                    "p99_ms": float(np.percentile(x, 99) * ms_per_iteration)}

        return {"ttft": stats(t), "itl": stats(g),
                "clock": f"iterations x {ms_per_iteration:.4f} ms measured per iteration"}

    def timed(self, arrival_ms: dict, end_ms, ttft_slo_ms: float, itl_slo_ms: float,
              wall_s: float) -> dict:
        """Latency on measured time: ``end_ms[i]`` is when iteration i's
        kernels ended and ``arrival_ms[seq]`` when the request arrived, on one
        clock.  TTFT = end of the first token's iteration - arrival; each
        inter-token latency = the gap between the ends of consecutive token
        iterations.  Goodput counts the output tokens of the requests that met
        both targets (TTFT within ``ttft_slo_ms`` and every inter-token gap
        within ``itl_slo_ms``) per second of ``wall_s``."""
        end_ms = np.asarray(end_ms, dtype=np.float64)
        ttft, gaps, good_tok, good_req, out_tok = [], [], 0, 0, 0
        for s, t in sorted(self.tokens.items()):
            if not t:
                continue
            e = end_ms[np.asarray(t)]
            f = float(e[0] - arrival_ms[s])
            g = np.diff(e)
            ttft.append(f)
            gaps.append(g)
            out_tok += len(t)
            if f <= ttft_slo_ms and (len(g) == 0 or float(g.max()) <= itl_slo_ms):
                good_tok += len(t)
                good_req += 1
        ttft = np.asarray(ttft)
        gaps = np.concatenate(gaps) if gaps else np.zeros(0)

        def stats(x):
            if len(x) == 0:
                return {"n": 0}
            return {"n": int(len(x)), "mean_ms": float(x.mean()), "min_ms": float(x.min()),
                    "p50_ms": float(np.percentile(x, 50)), "p99_ms": float(np.percentile(x, 99)),
                    "max_ms": float(x.max())}

        return {"ttft": stats(ttft), "itl": stats(gaps), "output_tokens": out_tok,
                "output_tokens_per_s": out_tok / wall_s,
                "goodput_tokens_per_s": good_tok / wall_s, "slo_met_requests": good_req,
                "slo": {"ttft_ms": ttft_slo_ms, "itl_ms": itl_slo_ms}}


def serve(run: LayerIterations, requests, ttft_slo_ms: float, itl_slo_ms: float,
          max_iters: int = 1_000_000, timeout_s: float = 120.0) -> dict:
    """Serves ``requests`` [(arrival_ms, id, prompt_len, output_len)] (in
    arrival order) through ``run`` on a live clock until every request has
    been released: before each iteration the requests whose arrival time
    has passed join the queue; when nothing runs or waits the host sleeps
    until the next arrival.  The end of every iteration is timed by an event
    on the compute stream; the host clock starts when a start event on that
    stream has completed, so arrival and end times share an origin (to the
    latency of that one synchronisation).  Returns the latency summary of
    ``LatencyLog.timed`` plus the iteration count and wall time (first
    arrival to the last iteration's end)."""
    import time

    log = LatencyLog()
    arrival = {}
    ends = []
    run.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    start.record(run.compute)
    start.synchronize()
    t0 = time.perf_counter()
    i, n, it = 0, len(requests), 0
    added = False
    while run.totals["finished"] < n:
        now = (time.perf_counter() - t0) * 1e3
        while i < n and requests[i][0] <= now:
            a, sid, p, o = requests[i]
            run.add(sid, p, o)
            log.add(it, sid, o)
            arrival[sid] = a
            added = True
            i += 1
        idle = it == 0 or (run.acc["running"] == 0 and run.acc["waiting"] == 0)
        if idle and not added:
            if i >= n:
                raise RuntimeError("serve: requests left unfinished with nothing queued")
            time.sleep(max(0.0, requests[i][0] / 1e3 - (time.perf_counter() - t0)))
            continue
        run.step()
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(run.compute)
        ends.append(ev)
        b = run.batch
        log.step(it, b.decode()[0], b.prefill()[0], b.emits())
        added = False
        it += 1
        if it >= max_iters or time.perf_counter() - t0 > timeout_s:
            raise RuntimeError(f"serve: {run.totals['finished']} of {n} requests finished "
                               f"after {it} iterations")
    run.synchronize()
    end_ms = np.array([start.elapsed_time(e) for e in ends])
    wall_s = float(end_ms[-1] - requests[0][0]) / 1e3
    out = log.timed(arrival, end_ms, ttft_slo_ms, itl_slo_ms, wall_s)
    out.update({"iterations": it, "wall_s": wall_s,
                "preemptions": run.totals["preempted"],
                "prefill_tokens": run.totals["prefill_tokens"],
                "decode_tokens": run.totals["decode_tokens"]})
    return out
