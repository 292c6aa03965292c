"""Pins of the oracle's continuous-batching scheduler: two hand-worked traces
and the invariants the texts state, on seeded random traces."""
import json
import os

import numpy as np

from oracle.allocator import BlockPool
from oracle.scheduler import Scheduler
from workloads import trace as make_trace

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run_golden(tr):
    pool = BlockPool(tr["num_blocks"], tr["block_size"])
    sch = Scheduler(pool, tr["max_running"], tr["prefill_budget"])
    for it, want in enumerate(tr["iterations"]):
        for sid, p, o in tr["arrivals"].get(str(it), []):
            sch.add(sid, p, o)
        b = sch.step()
        got = {"finished": b.finished, "admitted": b.admitted, "preempted": b.preempted,
               "decode": [list(x) for x in b.decode],
               "prefill": [[s, a, n, list(sl)] for s, a, n, sl in b.prefill],
               "free": pool.free_list(), "held": list(sch.held())}
        assert got == want, (tr["name"], it, got, want)


def test_hand_worked_traces():
    g = json.load(open(os.path.join(GOLDEN, "scheduler_traces.json")))
    for tr in g["traces"]:
        _run_golden(tr)


def _check_invariants(num_blocks, iters, lam, budget, max_running, seed):
    w = make_trace(seed=seed, iters=iters, lam=lam, prompt_median=60, prompt_sigma=1.0,
                   prompt_cap=400, out_mean=20, num_blocks=num_blocks)
    pool = BlockPool(num_blocks, 16)
    sch = Scheduler(pool, max_running, budget)
    produced = {}
    targets = {}
    for it in range(iters):
        for sid, p, o in w.arrivals[it]:
            sch.add(sid, p, o)
            targets[sid] = o
        b = sch.step()
        assert sum(n for _, _, n, _ in b.prefill) <= budget
        assert len(sch.running) <= max_running
        ids = [s for s, _, _ in b.decode] + [s for s, _, _, _ in b.prefill]
        assert len(ids) == len(set(ids))          # one unit per sequence per iteration
        for s, pos, slot in b.decode:
            t = pool.block_table(s)
            assert slot == t[pos // 16] * 16 + pos % 16
            assert pool.lengths[s] == pos + 1
        held = [x for t in pool.tables.values() for x in t]
        assert sorted(held + pool.free_list()) == list(range(num_blocks))
        for s in sch.running:
            assert pool.lengths[s.sid] == (s.known if s.in_prefill else s.cached_len())
        for s in sch.done:
            produced[s.sid] = s.decoded
    for sid, n in produced.items():
        assert n == targets[sid]
    return sch


def test_invariants_roomy_pool():
    sch = _check_invariants(num_blocks=4000, iters=300, lam=0.3, budget=64, max_running=16, seed=21)
    assert len(sch.done) > 20


def test_invariants_tiny_pool_forces_preemption():
    sch = _check_invariants(num_blocks=40, iters=400, lam=0.3, budget=64, max_running=16, seed=22)
    assert sum(s.preemptions for s in sch.done + sch.running + sch.waiting) > 0
    assert len(sch.done) > 5



_HELD = Scheduler.held


def _held_mutants():
    """Plausible mistakes in the accounting, each of which the hand-worked
    held values must catch."""
    def decoded_in_unwritten(self):
        b, a, u = _HELD(self)
        return b, a, u + sum(s.decoded for s in self.running if not s.in_prefill)

    def decode_phase_only(self):
        blocks = sum(len(self.pool.tables[s.sid]) for s in self.running if not s.in_prefill)
        tok = sum(self.pool.lengths[s.sid] for s in self.running if not s.in_prefill)
        return blocks, tok, 0

    def written_not_assigned(self):
        b, a, u = _HELD(self)
        return b, a - u, u

    def waiting_counted(self):
        b, a, u = _HELD(self)
        return b, a, u + sum(s.known for s in self.waiting)

    return [decoded_in_unwritten, decode_phase_only, written_not_assigned, waiting_counted]


def test_hand_worked_held_values_catch_accounting_mistakes(monkeypatch):
    """Mistakes planted in the oracle's accounting (on the CPU): counting
    decoded tokens as unwritten, dropping the prefill-phase sequences,
    counting only written tokens as assigned, charging the waiting queue."""
    g = json.load(open(os.path.join(GOLDEN, "scheduler_traces.json")))
    for mutant in _held_mutants():
        caught = False
        with monkeypatch.context() as m:
            m.setattr(Scheduler, "held", mutant)
            for tr in g["traces"]:
                try:
                    _run_golden(tr)
                except AssertionError:
                    caught = True
        assert caught, mutant.__name__


# -- prefix caching (ARTICLE §4.3) ------------------------------------------

def _run_prefix_golden(tr):
    pool = BlockPool(tr["num_blocks"], tr["block_size"])
    sch = Scheduler(pool, tr["max_running"], tr["prefill_budget"])
    for it, want in enumerate(tr["iterations"]):
        for sid, o, ids in tr["arrivals"].get(str(it), []):
            sch.add_prompt(sid, len(ids), o, ids)
        b = sch.step()
        got = {"finished": b.finished, "admitted": b.admitted, "preempted": b.preempted,
               "decode": [list(x) for x in b.decode],
               "prefill": [[s, a, n, list(sl)] for s, a, n, sl in b.prefill],
               "emits": [bool(e) for e in b.emits], "held": list(sch.held()),
               "free": pool.free_list(), "registered": pool.num_registered(),
               "prefix_hits": sch.prefix_hits}
        assert got == want, (it, got, want)


def test_prefix_caching_hand_worked_trace():
    _run_prefix_golden(json.load(open(os.path.join(GOLDEN, "prefix_sched_trace.json"))))


def _prefix_mutants():
    from oracle.allocator import OK, ceil_div

    def admit(full_prompt=False, discount=True, keep_shared=True):
        def _admit_prefix(self, out, s):
            bs = self.pool.block_size
            head = s.ids if full_prompt else s.ids[:s.prompt_len - 1]
            matched = self.pool.match_prefix(head)
            if self.pool.num_free() < ceil_div(s.known, bs) - (matched // bs if discount else 0):
                return False
            st, shared = self.pool.seq_create_prefix(s.sid, head)
            assert st == OK
            st, _ = self.pool.seq_append(s.sid, s.known - len(head))
            assert st == OK
            s.prefilled = shared if keep_shared else 0
            s.reg_blocks = shared // bs
            self.prefix_hits += shared
            self.waiting.pop(0)
            self.running.append(s)
            out.admitted.append(s.sid)
            return True
        return _admit_prefix

    def register_allocated(self):
        # blocks indexed once allocated rather than once computed
        bs = self.pool.block_size
        for s in self.running:
            if s.ids is None:
                continue
            nb = min(self.pool.lengths[s.sid], s.prompt_len) // bs
            if nb > s.reg_blocks:
                assert self.pool.seq_register_prefix(s.sid, s.ids[:nb * bs]) == OK
                s.reg_blocks = nb

    return [("_admit_prefix", admit(full_prompt=True), "whole prompt matched"),
            ("_admit_prefix", admit(discount=False), "fit ignores the shared blocks"),
            ("_admit_prefix", admit(keep_shared=False), "prefill restarts at 0"),
            ("_register_computed", register_allocated, "registered once allocated")]


def test_prefix_trace_catches_planted_mistakes(monkeypatch):
    """Mistakes planted in the oracle's prefix caching (on the CPU) each
    fail the hand-worked trace."""
    tr = json.load(open(os.path.join(GOLDEN, "prefix_sched_trace.json")))
    for attr, mutant, what in _prefix_mutants():
        with monkeypatch.context() as m:
            m.setattr(Scheduler, attr, mutant)
            try:
                _run_prefix_golden(tr)
                caught = False
            except AssertionError:
                caught = True
        assert caught, what


def test_prefix_caching_invariants_under_preemption():
    """Seeded traces whose prompts share a few system prefixes, on a pool
    small enough to preempt: every table holds distinct blocks, shared blocks
    are counted once per holder, the free list and the held blocks partition
    the pool, and each sequence's cached prefix is found again."""
    rng = np.random.default_rng(5)
    bs = 16
    prefixes = [rng.integers(0, 1000, n).tolist() for n in (40, 64, 100)]
    pool = BlockPool(24, bs)
    sch = Scheduler(pool, 8, 48)
    sid = 0
    hits = 0
    preempted = 0
    for it in range(300):
        for _ in range(rng.poisson(0.6)):
            ids = prefixes[rng.integers(0, 3)] + rng.integers(1000, 2000, rng.integers(1, 40)).tolist()
            sch.add_prompt(sid, len(ids), int(rng.integers(1, 80)), ids)
            sid += 1
        b = sch.step()
        preempted += len(b.preempted)
        assert sum(n for _, _, n, _ in b.prefill) <= 48
        for t in pool.tables.values():
            assert len(t) == len(set(t))
        held = {x for t in pool.tables.values() for x in t}
        assert sorted(list(held) + pool.free_list()) == list(range(24))
        for x in held:
            assert pool.refs[x] == sum(t.count(x) for t in pool.tables.values())
        for s in sch.running:
            assert pool.lengths[s.sid] == (s.known if s.in_prefill else s.cached_len())
        hits = sch.prefix_hits
    assert hits > 0 and sch.done and preempted > 0
