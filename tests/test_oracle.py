"""Pins of the CPU oracle against things other than itself.

Each test fixes a part of the oracle to an independent fact: a library
implementation of a storage format (torch's CPU casts), a hand-worked trace,
a dense attention written without block tables, a scalar brute force, a
closed form, or an invariance the definition implies.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import allocator as oa
from oracle import attention as oat
from oracle import cache as oc
from oracle import codecs
from oracle import fragmentation as ofr
from tests.prefix_truth import run_with_truth, seeded_cases

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------- codecs -----

def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_matches_torch_including_ties():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # force exact halfway cases (low half-word 0x8000) on a quarter of them
    bits[::4] = (bits[::4] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = codecs.bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encode_closed_forms():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even code (1.0)
    assert codecs.bf16_encode(np.float32(1.0 + 2.0 ** -8)) == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert codecs.bf16_encode(np.float32(1.0 + 3 * 2.0 ** -8)) == 0x3F82
    assert codecs.bf16_encode(np.float32(-2.0)) == 0xC000


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32) * 50,
        rng.uniform(-464, 464, 100_000).astype(np.float32),
        (rng.standard_normal(50_000) * 2.0 ** -8).astype(np.float32),     # subnormal range
        codecs.E4M3_TABLE[np.isfinite(codecs.E4M3_TABLE)].astype(np.float32),   # exact codes
    ])
    # exact midpoints between neighbouring positive codes
    v = codecs.E4M3_TABLE[:0x7F]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ours = codecs.e4m3_encode_sat(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturation_and_nan():
    big = np.array([448.0, 464.0, 465.0, 1e6, np.inf, -500.0, -np.inf], dtype=np.float32)
    got = codecs.e4m3_encode_sat(big)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    n = codecs.e4m3_encode_sat(np.array([np.nan], dtype=np.float32))
    assert np.isnan(codecs.e4m3_decode(n))[0]


def test_e4m3_quantize_round_trip_of_exact_multiples():
    # x = code_value * scale exactly, with a power-of-two scale: the stored
    # code must be the code itself.
    scale = np.float32(0.125)
    codes = np.array([c for c in range(256) if np.isfinite(codecs.E4M3_TABLE[c])], dtype=np.uint8)
    x = (codecs.E4M3_TABLE[codes] * 0.125).astype(np.float32)
    got = codecs.e4m3_quantize(x, scale)
    # +0 and -0 both decode to 0: compare values, and signs for nonzeros
    assert np.array_equal(codecs.e4m3_decode(got), codecs.E4M3_TABLE[codes])


# ---------------------------------------------------------- allocator -----

def test_allocator_hand_worked_trace():
    g = json.load(open(os.path.join(GOLDEN, "allocator_trace.json")))
    pool = oa.BlockPool(g["num_blocks"], g["block_size"], g["initial_free_order"])
    for step in g["steps"]:
        if step["op"] == "create":
            st_ = pool.seq_create(step["seq"], step["n"])
        elif step["op"] == "append":
            st_, slots = pool.seq_append(step["seq"], step["n"])
            if "slots" in step:
                assert slots == step["slots"], step
        else:
            st_ = pool.seq_release(step["seq"])
        assert st_ == step["status"], step
        assert pool.free_list() == step["free"], step
        if "table" in step:
            assert pool.block_table(step["seq"]) == step["table"], step


def run_sharing_step(pool, step):
    """Apply one step of the prefix-sharing fixture; returns its status."""
    if step["op"] == "create":
        return pool.seq_create(step["seq"], step["n"])
    if step["op"] == "append":
        st_, slots = pool.seq_append(step["seq"], step["n"])
        if "slots" in step:
            assert slots == step["slots"], step
        return st_
    if step["op"] == "share":
        st_, shared = pool.seq_share(step["seq"], step["src"], step["shared"], step["n"])
        if "shared_out" in step:
            assert shared == step["shared_out"], step
        return st_
    return pool.seq_release(step["seq"])


def test_prefix_sharing_hand_worked_trace():
    g = json.load(open(os.path.join(GOLDEN, "prefix_sharing_trace.json")))
    pool = oa.BlockPool(g["num_blocks"], g["block_size"], g["initial_free_order"])
    for step in g["steps"]:
        assert run_sharing_step(pool, step) == step["status"], step
        assert pool.free_list() == step["free"], step
        if "table" in step:
            assert pool.block_table(step["seq"]) == step["table"], step
        if "refs" in step:
            assert [pool.block_refs(b) for b in range(g["num_blocks"])] == step["refs"], step


def run_detection_step(pool, step):
    """(status, tokens in shared blocks or None) of one step."""
    if step["op"] == "create_prefix":
        return pool.seq_create_prefix(step["seq"], step["tokens"])
    if step["op"] == "register":
        return pool.seq_register_prefix(step["seq"], step["tokens"]), None
    return pool.seq_release(step["seq"]), None


def check_detection_trace(pool_cls):
    """Runs tests/golden/prefix_detection_trace.json (hand-worked) on a pool
    class with the oracle's interface; returns the first mismatch or None."""
    g = json.load(open(os.path.join(GOLDEN, "prefix_detection_trace.json")))
    pool = pool_cls(g["num_blocks"], g["block_size"], g["initial_free_order"])
    for i, step in enumerate(g["steps"]):
        status, shared = run_detection_step(pool, step)
        if status != step["status"]:
            return i, "status"
        if status == oa.OK and "shared_out" in step and shared != step["shared_out"]:
            return i, "shared tokens"
        if pool.free_list() != step["free"]:
            return i, "free list"
        if pool.num_registered() != step["registered"]:
            return i, "registered"
        if "table" in step and pool.block_table(step["seq"]) != step["table"]:
            return i, "table"
        if "refs" in step and [pool.block_refs(b) for b in range(g["num_blocks"])] != step["refs"]:
            return i, "refs"
    return None


def test_prefix_detection_hand_worked_trace():
    """ARTICLE 4.3 (prefix reuse, detection left to the scheduler): the
    oracle's detection against a trace worked by hand."""
    assert check_detection_trace(oa.BlockPool) is None


class _NoParent(oa.BlockPool):
    """Planted mistake: a block is found by its token ids alone."""

    def seq_create_prefix(self, seq, tokens):
        saved = self.index
        self.index = {(-1, k[1]): b for k, b in saved.items()}
        self._chain_off = True
        try:
            tokens = [int(t) for t in tokens]
            if seq in self.tables:
                return oa.ERR_EXISTS, 0
            bs, matched = self.block_size, []
            for i in range(len(tokens) // bs):
                b = self.index.get((-1, tuple(tokens[i * bs:(i + 1) * bs])))
                if b is None:
                    break
                matched.append(b)
            fresh = self._take(oa.ceil_div(len(tokens), bs) - len(matched))
            if fresh is None:
                return oa.ERR_NO_BLOCKS, 0
            for b in matched:
                self.refs[b] += 1
            self.tables[seq] = matched + fresh
            self.lengths[seq] = len(tokens)
            return oa.OK, len(matched) * bs
        finally:
            self.index = saved


class _KeepsFreed(oa.BlockPool):
    """Planted mistake: freed blocks stay in the index."""

    def _give_back(self, ids):
        saved = dict(self.content), dict(self.index)
        super()._give_back(ids)
        self.content, self.index = saved


class _NoStop(oa.BlockPool):
    """Planted mistake: the walk skips an unmatched block and goes on."""

    def seq_create_prefix(self, seq, tokens):
        tokens = [int(t) for t in tokens]
        if seq in self.tables:
            return oa.ERR_EXISTS, 0
        bs, table, parent, shared = self.block_size, [], -1, 0
        n = oa.ceil_div(len(tokens), bs)
        for i in range(n):
            b = self.index.get((parent, tuple(tokens[i * bs:(i + 1) * bs])))
            table.append(b)
            parent = b if b is not None else parent
        fresh = self._take(sum(b is None for b in table))
        if fresh is None:
            return oa.ERR_NO_BLOCKS, 0
        it = iter(fresh)
        table = [b if b is not None else next(it) for b in table]
        for b in table:
            if b not in fresh:
                self.refs[b] += 1
                shared += bs
        self.tables[seq] = table
        self.lengths[seq] = len(tokens)
        return oa.OK, shared


@pytest.mark.parametrize("cls", [_NoParent, _KeepsFreed, _NoStop])
def test_prefix_detection_trace_catches_planted_mistakes(cls):
    assert check_detection_trace(cls) is not None


share_ops = st.lists(st.tuples(st.sampled_from(["create", "append", "release", "share"]),
                               st.integers(0, 5), st.integers(0, 5), st.integers(0, 70),
                               st.integers(0, 70)), max_size=60)


@settings(max_examples=200, deadline=None)
@given(share_ops, st.integers(0, 40))
def test_prefix_sharing_invariants(oplist, nblocks):
    """Every block is counted once per table holding it; the free blocks are
    exactly those no table holds, each once; shared blocks are full, so no
    position a sequence may still write lies in a block another table holds;
    failed calls change nothing."""
    pool = oa.BlockPool(nblocks, 16)
    for op, seq, src, n, shared in oplist:
        before = (pool.free_list(), {k: list(v) for k, v in pool.tables.items()},
                  dict(pool.lengths), list(pool.refs))
        if op == "create":
            st_ = pool.seq_create(seq, n)
        elif op == "append":
            st_, _ = pool.seq_append(seq, n)
        elif op == "share":
            st_, got = pool.seq_share(seq, src, shared, max(n, shared))
            if st_ == oa.OK:
                assert got == (shared // 16) * 16
                assert pool.tables[seq][:shared // 16] == before[1][src][:shared // 16]
        else:
            st_ = pool.seq_release(seq)
        if st_ != oa.OK:
            assert (pool.free_list(), {k: list(v) for k, v in pool.tables.items()},
                    dict(pool.lengths), list(pool.refs)) == before
        counts = [0] * nblocks
        for t in pool.tables.values():
            assert len(t) == len(set(t))
            for b in t:
                counts[b] += 1
        assert counts == pool.refs
        assert sorted(pool.free_list()) == [b for b in range(nblocks) if counts[b] == 0]
        for s, t in pool.tables.items():
            assert len(t) == -(-pool.lengths[s] // 16)
            # a sequence writes only at positions >= its length; the block
            # holding its next position, if it has one, is its own
            nxt = pool.lengths[s] // 16
            if nxt < len(t):
                assert pool.refs[t[nxt]] == 1


ops = st.lists(st.tuples(st.sampled_from(["create", "append", "release"]),
                         st.integers(0, 5), st.integers(0, 70)), max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops, st.integers(0, 40), st.randoms(use_true_random=False))
def test_allocator_invariants(oplist, nblocks, rnd):
    order = list(range(nblocks))
    rnd.shuffle(order)
    pool = oa.BlockPool(nblocks, 16, order)
    expect_free = list(order)
    for op, seq, n in oplist:
        before = (pool.free_list(), {k: list(v) for k, v in pool.tables.items()}, dict(pool.lengths))
        if op == "create":
            st_ = pool.seq_create(seq, n)
        elif op == "append":
            st_, _ = pool.seq_append(seq, n)
        else:
            st_ = pool.seq_release(seq)
        if st_ != oa.OK:
            after = (pool.free_list(), {k: list(v) for k, v in pool.tables.items()}, dict(pool.lengths))
            assert after == before            # failed calls change nothing
        held = [b for t in pool.tables.values() for b in t]
        assert len(held) == len(set(held))
        assert sorted(held + pool.free_list()) == list(range(nblocks))
        for s, t in pool.tables.items():
            assert len(t) == -(-pool.lengths[s] // 16)
        # FIFO: the free list is always a suffix of what was taken plus the
        # released tables appended in order
        if op == "create" and st_ == oa.OK:
            k = -(-n // 16)
            assert pool.tables[seq] == expect_free[:k]
            expect_free = expect_free[k:]
        elif op == "release" and st_ == oa.OK:
            expect_free = expect_free + before[1][seq]
        elif op == "append" and st_ == oa.OK:
            k = len(pool.tables[seq]) - len(before[1][seq])
            assert pool.tables[seq][len(before[1][seq]):] == expect_free[:k]
            expect_free = expect_free[k:]
        assert pool.free_list() == expect_free


def test_slot_formula():
    pool = oa.BlockPool(8, 16, [5, 2, 7, 0, 1, 3, 4, 6])
    assert pool.seq_create(9, 40) == oa.OK
    assert pool.block_table(9) == [5, 2, 7]
    assert pool.slots(9, 0, 40) == ([5 * 16 + i for i in range(16)] + [2 * 16 + i for i in range(16)]
                                    + [7 * 16 + i for i in range(8)])


# ------------------------------------------------------------ attention ---

def _dense_reference(q, k, v, sm_scale):
    """Attention on contiguous arrays via einsum and log-sum-exp (a route that
    uses no block table and a differently written softmax)."""
    z = np.einsum("hd,ld->hl", q, k) * sm_scale
    lse = np.log(np.sum(np.exp(z - z.max(axis=1, keepdims=True)), axis=1, keepdims=True)) + z.max(axis=1, keepdims=True)
    return np.einsum("hl,ld->hd", np.exp(z - lse), v)


def _paged_setup(rng, lengths, h_kv, d, dtype="f32", nblocks=None, bs=16):
    need = sum(-(-L // bs) for L in lengths)
    nblocks = nblocks or need + 3
    pool = oa.BlockPool(nblocks, bs, rng.permutation(nblocks).tolist())
    kc, vc = oc.new_cache(nblocks, h_kv, bs, d, dtype)
    dense = []
    for s, L in enumerate(lengths):
        assert pool.seq_create(s, int(L)) == oa.OK
        k = rng.standard_normal((L, h_kv, d)).astype(np.float32)
        v = rng.standard_normal((L, h_kv, d)).astype(np.float32)
        oc.cache_write(kc, vc, k, v, pool.slots(s, 0, L), "f32", "f32")
        dense.append((k.astype(np.float64), v.astype(np.float64)))
    tables, lens = pool.pack(range(len(lengths)), max(-(-L // bs) for L in lengths))
    return pool, kc, vc, np.array(tables), np.array(lens), dense


def test_decode_matches_dense_contiguous_attention():
    rng = np.random.default_rng(3)
    lengths = [1, 15, 16, 17, 200, 333]
    h_q, h_kv, d = 8, 2, 32
    _, kc, vc, tables, lens, dense = _paged_setup(rng, lengths, h_kv, d)
    q = rng.standard_normal((len(lengths), h_q, d))
    sm = float(np.float32(1 / math.sqrt(d)))
    out = oat.decode(q, kc, vc, tables, lens, h_kv, sm, "f32")
    for s in range(len(lengths)):
        k, v = dense[s]
        for h in range(h_q):
            kh = h // (h_q // h_kv)
            ref = _dense_reference(q[s, h][None], k[:, kh], v[:, kh], sm)[0]
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12, atol=1e-14)


def test_decode_scalar_brute_force():
    rng = np.random.default_rng(4)
    lengths = [3, 20]
    _, kc, vc, tables, lens, dense = _paged_setup(rng, lengths, 1, 4)
    q = rng.standard_normal((2, 2, 4))
    out = oat.decode(q, kc, vc, tables, lens, 1, 0.5, "f32")
    for s, L in enumerate(lengths):
        k, v = dense[s]
        for h in range(2):
            z = [0.5 * sum(q[s, h, i] * k[p, 0, i] for i in range(4)) for p in range(L)]
            m = max(z)
            e = [math.exp(x - m) for x in z]
            tot = sum(e)
            ref = [sum(e[p] * v[p, 0, i] for p in range(L)) / tot for i in range(4)]
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12, atol=1e-15)


def test_decode_invariant_under_block_permutation():
    rng = np.random.default_rng(5)
    lengths = [40, 7, 64]
    _, kc, vc, tables, lens, _ = _paged_setup(rng, lengths, 2, 16, nblocks=20)
    q = rng.standard_normal((3, 4, 16))
    base = oat.decode(q, kc, vc, tables, lens, 2, 0.25, "f32")
    perm = rng.permutation(20)              # block b moves to perm[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    moved = oat.decode(q, kc2, vc2, t2, lens, 2, 0.25, "f32")
    assert np.array_equal(base, moved)


def test_decode_closed_forms():
    rng = np.random.default_rng(6)
    d = 8
    # L = 1: the output is the single value row, exactly
    _, kc, vc, tables, lens, dense = _paged_setup(rng, [1], 1, d)
    q = rng.standard_normal((1, 1, d))
    out = oat.decode(q, kc, vc, tables, lens, 1, 0.3, "f32")
    assert np.array_equal(out[0, 0], dense[0][1][0, 0])
    # q = 0: uniform weights, output = mean of V
    _, kc, vc, tables, lens, dense = _paged_setup(rng, [37], 1, d)
    out = oat.decode(np.zeros((1, 1, d)), kc, vc, tables, lens, 1, 0.3, "f32")
    np.testing.assert_allclose(out[0, 0], dense[0][1][:, 0].mean(axis=0), rtol=1e-12)
    # constant V: output = that constant
    vc[:] = np.float32(0.75)
    out = oat.decode(q, kc, vc, tables, lens, 1, 0.3, "f32")
    np.testing.assert_allclose(out[0, 0], 0.75, rtol=1e-14)
    # one dominant key: output within e^-gap of its value row
    _, kc, vc, tables, lens, dense = _paged_setup(rng, [50], 1, d)
    qd = np.zeros((1, 1, d))
    qd[0, 0, 0] = 1.0
    kc[:, :, 0, :, 0] = 0.0              # key dim 0 of every token (layout [b][h][d/x][o][x])
    b, o = tables[0][33 // 16], 33 % 16
    kc[b, 0, 0, o, 0] = 40.0             # score gap 40 * scale(1.0)
    out = oat.decode(qd, kc, vc, tables, lens, 1, 1.0, "f32")
    np.testing.assert_allclose(out[0, 0], dense[0][1][33, 0], atol=50 * math.exp(-40) * 10)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(7)
    lengths = [30, 45]
    h_q, h_kv, d = 6, 2, 8
    _, kc, vc, tables, lens, _ = _paged_setup(rng, lengths, h_kv, d)
    q = rng.standard_normal((2, h_q, d))
    gqa = oat.decode(q, kc, vc, tables, lens, h_kv, 0.4, "f32")
    g = h_q // h_kv
    kc_rep = np.repeat(kc, g, axis=1)
    vc_rep = np.repeat(vc, g, axis=1)
    mha = oat.decode(q, kc_rep, vc_rep, tables, lens, h_q, 0.4, "f32")
    # same mathematics; BLAS may group the rows differently, so allow rounding
    np.testing.assert_allclose(gqa, mha, rtol=1e-13, atol=1e-15)
    # and a wrong head map (h % H_kv instead of h // G) is detectably different
    wrong = np.concatenate([kc[:, [h % h_kv]] for h in range(h_q)], axis=1)
    wrongv = np.concatenate([vc[:, [h % h_kv]] for h in range(h_q)], axis=1)
    bad = oat.decode(q, wrong, wrongv, tables, lens, h_q, 0.4, "f32")
    assert np.abs(bad - gqa).max() > 1e-3


def test_prefill_chunks_equal_one_causal_attention_and_decode_rows():
    rng = np.random.default_rng(8)
    P, chunk = 96, 32
    h_q, h_kv, d = 4, 2, 16
    _, kc, vc, tables, lens, dense = _paged_setup(rng, [P], h_kv, d)
    q = rng.standard_normal((P, h_q, d))
    sm = 0.25
    k, v = dense[0]
    for c in range(P // chunk):
        rows = oat.prefill_chunk(q[c * chunk:(c + 1) * chunk], c * chunk, kc, vc, tables[0], h_kv, sm, "f32")
        for i in range(chunk):
            p = c * chunk + i
            for h in range(h_q):
                kh = h // (h_q // h_kv)
                ref = _dense_reference(q[p, h][None], k[:p + 1, kh], v[:p + 1, kh], sm)[0]
                np.testing.assert_allclose(rows[i, h], ref, rtol=1e-12, atol=1e-14)
    # decode of position p with context p+1 equals prefill row p
    p = 70
    dec = oat.decode(q[p][None], kc, vc, tables[:1], np.array([p + 1]), h_kv, sm, "f32")
    row = oat.prefill_chunk(q[64:96], 64, kc, vc, tables[0], h_kv, sm, "f32")[p - 64]
    np.testing.assert_allclose(dec[0], row, rtol=1e-13, atol=1e-15)


def test_fp8_cache_decodes_to_scaled_codes():
    rng = np.random.default_rng(9)
    x = codecs.bf16_encode(rng.standard_normal((20, 1, 16)).astype(np.float32))
    pool = oa.BlockPool(2, 16, [1, 0])
    pool.seq_create(0, 20)
    kc, vc = oc.new_cache(2, 1, 16, 16, "fp8")
    ks, vs = 0.01, 0.02
    oc.cache_write(kc, vc, x, x, pool.slots(0, 0, 20), "bf16", "fp8", ks, vs)
    k, v = oat.gather(kc, vc, pool.block_table(0), 20, 0, "fp8", ks, vs)
    src = codecs.bf16_decode(x)[:, 0]
    # quantisation error of e4m3 with RNE: at most half a unit in the last
    # place of the code's binade (relative 2^-4) or half the smallest
    # subnormal step
    err = np.abs(k - src)
    bound = np.maximum(np.abs(src) * 2.0 ** -4, 2.0 ** -10 * ks) * 1.0001
    assert np.all(err <= bound)
    assert np.all(np.abs(v - src) <= np.maximum(np.abs(src) * 2.0 ** -4, 2.0 ** -10 * vs) * 1.0001)


# -------------------------------------------------------- fragmentation ---

def test_fragmentation_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "fragmentation.json")))
    w = ofr.contiguous_waste([g["used"]], g["reserved"])
    assert round(100 * w) == g["waste_percent_rounded"]


def test_paged_waste_closed_form_and_exercise():
    assert ofr.paged_waste([17]) == 15 / 32
    assert ofr.paged_waste([16, 32]) == 0.0
    # LESSON exercise 4: 1000 requests, mean 1500, sd 600
    rng = np.random.default_rng(11)
    s2 = math.log(1 + (600 / 1500) ** 2)
    L = np.ceil(rng.lognormal(math.log(1500) - s2 / 2, math.sqrt(s2), 1000)).astype(np.int64)
    paged = ofr.paged_waste(L)
    contiguous = ofr.contiguous_waste(L)
    exact = float(np.sum(16 * np.ceil(L / 16) - L)) / float(np.sum(16 * np.ceil(L / 16)))
    assert paged == pytest.approx(exact, rel=1e-12)
    assert 0.003 < paged < 0.007          # about 7.5 wasted tokens of ~1508 held
    assert abs(contiguous - (1 - L.mean() / 8192)) < 1e-12
    assert 0.80 < contiguous < 0.83


# -- prefix retention (an extension beyond the pages; off by default) --------

def run_retention_step(pool, step):
    """The observable results of one step of prefix_retention_trace.json."""
    op = step["op"]
    res = {}
    if op == "retention":
        res["status"] = pool.set_prefix_retention(step["on"])
    elif op == "create_prefix":
        res["status"], res["shared_out"] = pool.seq_create_prefix(step["seq"], step["tokens"])
    elif op == "register":
        res["status"] = pool.seq_register_prefix(step["seq"], step["tokens"])
    elif op == "release":
        res["status"] = pool.seq_release(step["seq"])
    elif op == "create":
        res["status"] = pool.seq_create(step["seq"], step["n"])
    else:
        res["status"] = oa.OK
        res["matched"], res["matched_retained"] = pool.match_prefix(step["tokens"],
                                                                     with_retained=True)
    return res


def check_retention_trace(pool_cls):
    """Runs tests/golden/prefix_retention_trace.json (hand-worked) on a pool
    class with the oracle's interface; returns the first mismatch or None."""
    g = json.load(open(os.path.join(GOLDEN, "prefix_retention_trace.json")))
    pool = pool_cls(g["num_blocks"], g["block_size"], g["initial_free_order"])
    for i, step in enumerate(g["steps"]):
        try:
            res = run_retention_step(pool, step)
        except AssertionError:
            return i, "raised"
        res["free"] = pool.free_list()
        res["registered"] = pool.num_registered()
        res["retained"] = pool.num_retained()
        if "table" in step:
            res["table"] = pool.block_table(step["seq"])
        if "refs" in step:
            res["refs"] = [pool.block_refs(b) for b in range(g["num_blocks"])]
        for k, v in step.items():
            if k in res and res[k] != v and not (k == "shared_out" and res["status"] != oa.OK):
                return i, k
    return None


def test_prefix_retention_hand_worked_trace():
    assert check_retention_trace(oa.BlockPool) is None


class _NoRevive(oa.BlockPool):
    """Planted mistake: a retained block found by a lookup is used but stays
    in the retained list."""

    def seq_create_prefix(self, seq, tokens):
        saved = dict(self.retained)
        st, shared = super().seq_create_prefix(seq, tokens)
        if st == oa.OK:
            for b in saved:
                if b in self.tables[seq] and b not in self.retained:
                    self.retained[b] = None
        return st, shared


class _EvictNewest(oa.BlockPool):
    """Planted mistake: the most recently retained block is evicted first."""

    def _take(self, n):
        if self.num_free() < n:
            return None
        ids = []
        for _ in range(n):
            if self.free:
                b = self.free.popleft()
            else:
                b, _ = self.retained.popitem(last=True)
                self._unregister(b)
            ids.append(b)
        for b in ids:
            self.refs[b] = 1
        return ids


class _RetainedFirst(oa.BlockPool):
    """Planted mistake: fresh blocks come from the retained blocks first."""

    def _take(self, n):
        if self.num_free() < n:
            return None
        ids = []
        for _ in range(n):
            if self.retained:
                b, _ = self.retained.popitem(last=False)
                self._unregister(b)
            else:
                b = self.free.popleft()
            ids.append(b)
        for b in ids:
            self.refs[b] = 1
        return ids


class _RevivedCountFree(oa.BlockPool):
    """Planted mistake: the fit check counts the matched retained blocks as
    fresh blocks too."""

    def seq_create_prefix(self, seq, tokens):
        tokens = [int(t) for t in tokens]
        if seq in self.tables:
            return oa.ERR_EXISTS, 0
        bs, matched, parent = self.block_size, [], -1
        for i in range(len(tokens) // bs):
            b = self.index.get((parent, tuple(tokens[i * bs:(i + 1) * bs])))
            if b is None:
                break
            matched.append(b)
            parent = b
        if oa.ceil_div(len(tokens), bs) - len(matched) > self.num_free():
            return oa.ERR_NO_BLOCKS, 0
        for b in matched:
            if self.refs[b] == 0:
                del self.retained[b]
        fresh = self._take(oa.ceil_div(len(tokens), bs) - len(matched))
        assert fresh is not None
        for b in matched:
            self.refs[b] += 1
        self.tables[seq] = matched + fresh
        self.lengths[seq] = len(tokens)
        return oa.OK, len(matched) * bs


class _RetainInTableOrder(oa.BlockPool):
    """Planted mistake: a release retains its blocks in table order, so the
    head of a chain is evicted first and strands the rest."""

    def _give_back(self, ids):
        for b in ids:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                if self.retain and b in self.content:
                    self.retained[b] = None
                    continue
                self._unregister(b)
                self.free.append(b)


def test_prefix_retention_trace_catches_planted_mistakes():
    for cls in (_NoRevive, _EvictNewest, _RetainedFirst, _RevivedCountFree, _RetainInTableOrder):
        assert check_retention_trace(cls) is not None, cls.__name__


def test_retention_never_shares_a_block_computed_under_another_prefix():
    """Two blocks, 2-token blocks: the prompt a a b b is computed, registered
    and released with retention on; the next prompt (c c) needs one fresh
    block, which must be the retained tail (b b), not the head (a a).  Taking
    the head leaves the tail's key naming the head's id, which c c then
    occupies, so c c b b would be handed the b b block computed after a a."""
    ops = [("retention", True), ("create", 1, [0, 0, 1, 1]), ("register", 1, 4),
           ("release", 1), ("create", 2, [2, 2]), ("register", 2, 4),
           ("create", 3, [2, 2, 1, 1])]
    run_with_truth(oa.BlockPool(2, 2), ops)
    for cls in (_RetainInTableOrder, _EvictNewest):
        with pytest.raises(AssertionError):
            run_with_truth(cls(2, 2), ops)


def test_prefix_blocks_always_hold_their_own_prefix():
    """6000 seeded random runs: prompts over a two-letter alphabet, appends,
    registrations of any computed prefix, releases and retention switched on
    and off, on pools small enough that retained blocks are evicted all the
    time.  No sequence is ever handed a block computed under a different
    prefix; the same runs on the two planted eviction-order mistakes fail
    (each in roughly one run of a hundred and fifty)."""
    cases = seeded_cases()
    for ops, nblocks in cases:
        run_with_truth(oa.BlockPool(nblocks, 2), ops)
    for cls in (_RetainInTableOrder, _EvictNewest):
        failed = 0
        for ops, nblocks in cases:
            try:
                run_with_truth(cls(nblocks, 2), ops)
            except AssertionError:
                failed += 1
        assert failed > 0, cls.__name__
