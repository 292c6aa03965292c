"""The four schedules of the LESSON's simulator ("Use It": one request at a
time, padded static batches, iteration-level admission without chunking,
and chunked continuous batching) in the C scheduler (pa_sched_create_mode):
bit-exact against the oracle scheduler on random traces, and both pinned to
what the descriptions fix independently of either implementation: a
hand-worked static batch, the service recurrence of one-at-a-time
serving, the shape of every static batch, the reduction of the unchunked
schedule to the chunked one when no budget binds, and whole-prompt prefill.
Also the measured-clock latency summary on a hand-worked case.  CPU only."""
import numpy as np
import pytest

import paged_kv_cache_host_amd._pa as pa
from paged_kv_cache_host_amd.iteration import LatencyLog
from workloads import trace as make_trace

from oracle.allocator import BlockPool
from oracle.scheduler import Scheduler
from test_host_scheduler import CSide, _compare, _oracle_batch


class OSide:
    """The oracle scheduler behind CSide's interface, so that every pin
    below holds the oracle and the C scheduler to the same facts."""

    def __init__(self, num_blocks, max_running, budget, mode="chunked"):
        self.pool = BlockPool(num_blocks, 16)
        self.sch = Scheduler(self.pool, max_running, budget, mode=mode)

    def add(self, sid, p, o):
        self.sch.add(sid, p, o)

    def step(self):
        return _oracle_batch(self.sch.step())

    def free_list(self):
        return list(self.pool.free_list())

    def close(self):
        pass


side = pytest.mark.parametrize("make", [CSide, OSide], ids=["c", "oracle"])


def _drive(c, w, iters=None):
    """Runs the C scheduler over a trace; returns the per-iteration batches."""
    out = []
    for it in range(iters or w.iters):
        for sid, p, n in w.arrivals[it]:
            c.add(sid, p, n)
        out.append(c.step())
    return out


@pytest.mark.parametrize("mode,budget,max_running", [("continuous", 64, 16),
                                                     ("static", 1600, 8),
                                                     ("naive", 64, 16)])
@pytest.mark.parametrize("num_blocks", [4000, 40])
def test_modes_match_oracle(mode, budget, max_running, num_blocks):
    w = make_trace(seed=41, iters=300, lam=0.3, prompt_median=60, prompt_sigma=1.0,
                   prompt_cap=400, out_mean=20, num_blocks=num_blocks)
    totals, o = _compare(w, max_running, budget, mode=mode)
    assert totals["decode"] > 100 and len(o.done) > 5
    if num_blocks == 40 and mode != "naive":
        assert totals["preempted"] > 0


@side
def test_static_hand_worked(make):
    """Two slots, budget 100, a 100-block FIFO pool; A (prompt 20, 2 tokens),
    B (40, 1) and C (10, 1) arrive together.  Iteration 0 forms the batch
    [A, B] padded to 40 tokens (2 x 40 <= 100) and prefills both whole (A:
    blocks 0-2, B: 3-5); iteration 1 decodes both at position 40 (B's token
    is padding: it already has its one token); iteration 2 releases the
    batch (A's blocks then B's go to the back of the free list) and forms
    [C], which takes block 6."""
    c = make(100, 2, 100, mode="static")
    for sid, p, n in ((0, 20, 2), (1, 40, 1), (2, 10, 1)):
        c.add(sid, p, n)
    b0, b1, b2, b3 = (c.step() for _ in range(4))
    assert b0["admitted"] == [0, 1] and b0["decode"] == []
    assert b0["prefill"] == [[0, 0, 40, list(range(0, 40))], [1, 0, 40, list(range(48, 88))]]
    assert b0["emits"] == [True, True]
    assert b1["decode"] == [[0, 40, 40], [1, 40, 88]] and b1["prefill"] == []
    assert b1["finished"] == [] and b1["admitted"] == []
    assert b2["finished"] == [0, 1] and b2["admitted"] == [2]
    assert b2["prefill"] == [[2, 0, 10, list(range(96, 106))]] and b2["decode"] == []
    assert b3["finished"] == [2]
    assert c.free_list() == list(range(7, 100)) + [0, 1, 2, 3, 4, 5, 6]
    c.close()


@side
def test_naive_service_recurrence(make):
    """One request at a time on a roomy pool: request k is admitted at
    a_k = max(arrival_k, a_(k-1) + P_(k-1) + t_(k-1) - 1), where P =
    ceil(prompt / budget) prefill iterations and t its target (its last token
    comes out at a + P + t - 2, and it is released one iteration later,
    where the next one is admitted)."""
    w = make_trace(seed=43, iters=600, lam=0.05, prompt_median=60, prompt_sigma=1.0,
                   prompt_cap=400, out_mean=8, num_blocks=4000)
    B = 64
    c = make(w.num_blocks, 16, B, mode="naive")
    batches = _drive(c, w)
    c.close()
    admitted_at = {s: it for it, b in enumerate(batches) for s in b["admitted"]}
    reqs = [(it, sid, p, n) for it in range(w.iters) for sid, p, n in w.arrivals[it]]
    prev_end = 0
    checked = 0
    for arr, sid, p, n in reqs:
        a = max(arr, prev_end)
        if a >= w.iters:
            break
        assert admitted_at[sid] == a, sid
        prev_end = a + -(-p // B) + n - 1
        checked += 1
    assert checked > 10
    for b in batches:
        assert len(b["decode"]) + len({x[0] for x in b["prefill"]}) <= 1


@side
def test_static_batch_shape(make):
    """Every static batch on a roomy pool: formed only when nothing runs, from
    the heads of the queue; its prompts all prefilled, whole and padded to the
    longest, in the iteration that forms it (members x longest <= budget); the
    batch released together exactly max(target) iterations later."""
    w = make_trace(seed=44, iters=500, lam=0.3, prompt_median=60, prompt_sigma=1.0,
                   prompt_cap=400, out_mean=10, num_blocks=8000)
    R, B = 8, 1600
    c = make(w.num_blocks, R, B, mode="static")
    batches = _drive(c, w)
    c.close()
    req = {sid: (p, n) for row in w.arrivals for sid, p, n in row}
    running = set()
    n_batches = 0
    for it, b in enumerate(batches):
        running -= set(b["finished"])
        if b["finished"]:
            assert not running, it          # released together
        if b["admitted"]:
            assert not running, it
            members = b["admitted"]
            width = max(req[s][0] for s in members)
            assert len(members) <= R and len(members) * width <= B
            assert [x[0] for x in b["prefill"]] == members
            assert all(x[1] == 0 and x[2] == width for x in b["prefill"])
            assert all(b["emits"])
            end = it + max(req[s][1] for s in members)
            if end < len(batches):
                assert sorted(batches[end]["finished"]) == sorted(members), it
            running |= set(members)
            n_batches += 1
        for s, pos, _ in b["decode"]:
            assert s in running
    assert n_batches > 5


@side
def test_continuous_reduces_to_chunked_when_budget_never_binds(make):
    """With a budget above every iteration's prompt tokens, whole-prompt
    admission and chunked admission make the same decisions."""
    w = make_trace(seed=45, iters=300, lam=0.3, prompt_median=60, prompt_sigma=1.0,
                   prompt_cap=400, out_mean=20, num_blocks=4000)
    big = 16 * 400 + 1
    a, b = make(w.num_blocks, 16, big, mode="continuous"), make(w.num_blocks, 16, big)
    assert _drive(a, w) == _drive(b, w)
    a.close()
    b.close()


@side
def test_continuous_prefills_whole_prompts(make):
    """A binding budget: every prompt that fits the budget is prefilled in one
    slice, in the iteration that admits it; longer ones are sliced at the
    budget in iterations with no other prefill (their last slice may leave
    room for whole prompts after it); no iteration exceeds it."""
    w = make_trace(seed=46, iters=300, lam=0.5, prompt_median=60, prompt_sigma=1.0,
                   prompt_cap=400, out_mean=20, num_blocks=4000)
    B = 128
    c = make(w.num_blocks, 16, B, mode="continuous")
    batches = _drive(c, w)
    c.close()
    req = {sid: p for row in w.arrivals for sid, p, _ in row}
    long_seen = short_seen = 0
    for b in batches:
        assert sum(x[2] for x in b["prefill"]) <= B
        for s, start, n, _ in b["prefill"]:
            if req[s] <= B:
                assert start == 0 and n == req[s] and s in b["admitted"]
                short_seen += 1
            else:
                # a full-budget slice alone, or the last slice, ahead of any
                # prompts admitted into the rest of the budget
                assert b["prefill"][0][0] == s
                assert (n == B and len(b["prefill"]) == 1) or start + n == req[s]
                long_seen += 1
    assert short_seen > 50 and long_seen > 0


def test_mode_arguments():
    st, pool = pa.pa_pool_create(10, 16, None)
    pa.check(st)
    assert pa.pa_sched_create_mode(pool, "static", 4, 0, 16)[0] == pa.PA_ERR_INVALID
    assert pa.pa_sched_create_mode(pool, "continuous", 4, 0, 16)[0] == pa.PA_ERR_INVALID
    st, h = pa.pa_sched_create_mode(pool, "chunked", 4, 0, 16)
    assert st == pa.PA_OK
    pa.pa_sched_destroy(h)
    assert pa._lib.pa_sched_create_mode(pool, 7, 4, 64, 16, pa.C.byref(pa._vp())) == \
        pa.PA_ERR_INVALID
    pa.pa_pool_destroy(pool)


def test_timed_latency_hand_worked():
    """Requests 0 (3 tokens) and 1 (2 tokens) on iteration end times 1, 2, 4,
    4.5, 8 ms: request 0 arrives at 0.5 ms, tokens from iterations 0, 1 and
    3 -> TTFT 0.5, gaps 1 and 2.5; request 1 arrives at 1.0, tokens from
    iterations 2 and 4 -> TTFT 3, gap 4.  With targets TTFT <= 2 and gaps
    <= 2.5 only request 0 meets both: goodput 3 tokens / 0.01 s."""
    log = LatencyLog()
    log.add(0, 0, 3)
    log.add(1, 1, 2)
    log.step(0, [], [0], [1])
    log.step(1, [0], [1], [0])
    log.step(2, [], [1], [1])
    log.step(3, [0], [], [])
    log.step(4, [1, 0], [], [])       # request 0 is past its target here
    r = log.timed({0: 0.5, 1: 1.0}, [1.0, 2.0, 4.0, 4.5, 8.0], 2.0, 2.5, 0.01)
    assert r["ttft"]["n"] == 2 and r["ttft"]["mean_ms"] == pytest.approx(1.75)
    assert r["ttft"]["max_ms"] == pytest.approx(3.0) and r["ttft"]["min_ms"] == pytest.approx(0.5)
    assert r["itl"]["n"] == 3 and r["itl"]["max_ms"] == pytest.approx(4.0)
    assert r["itl"]["mean_ms"] == pytest.approx(7.5 / 3)
    assert r["output_tokens"] == 5 and r["slo_met_requests"] == 1
    assert r["goodput_tokens_per_s"] == pytest.approx(300.0)
    assert r["output_tokens_per_s"] == pytest.approx(500.0)
