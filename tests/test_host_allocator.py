"""libpa's host block pool (C++) against the oracle allocator, bit-exactly,
plus the library's exported symbols.  CPU only: no kernel is launched."""
import json
import os
import re
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import paged_kv_cache_host_amd as pa
import paged_kv_cache_host_amd._pa  # noqa: F401  (pa._pa: library path and handle)
from oracle import allocator as oa
from tests.prefix_truth import run_with_truth, seeded_cases

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 20
    out = subprocess.run(["nm", "-D", "--defined-only", pa._pa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    # and the binding covers the same set
    assert sorted(pa.EXPORTED) == names


def _state(pool):
    st_, free = pa.pa_pool_free_list(pool)
    assert st_ == pa.PA_OK
    return list(free)


def test_golden_trace_through_c_abi():
    g = json.load(open(os.path.join(GOLDEN, "allocator_trace.json")))
    st_, pool = pa.pa_pool_create(g["num_blocks"], g["block_size"], g["initial_free_order"])
    assert st_ == pa.PA_OK
    try:
        for step in g["steps"]:
            if step["op"] == "create":
                s = pa.pa_seq_create(pool, step["seq"], step["n"])
            elif step["op"] == "append":
                s, slots = pa.pa_seq_append(pool, step["seq"], step["n"])
                if "slots" in step:
                    assert list(slots) == step["slots"]
            else:
                s = pa.pa_seq_release(pool, step["seq"])
            assert s == step["status"], (step, pa.pa_last_error())
            assert _state(pool) == step["free"]
            if "table" in step:
                assert list(pa.pa_seq_block_table(pool, step["seq"])[1]) == step["table"]
    finally:
        pa.pa_pool_destroy(pool)


ops = st.lists(st.tuples(st.sampled_from(["create", "append", "release", "pack"]),
                         st.integers(0, 6), st.integers(0, 90)), max_size=80)


@settings(max_examples=300, deadline=None)
@given(ops, st.integers(0, 48), st.randoms(use_true_random=False))
def test_bit_exact_against_oracle(oplist, nblocks, rnd):
    order = list(range(nblocks))
    rnd.shuffle(order)
    ref = oa.BlockPool(nblocks, 16, order)
    st_, pool = pa.pa_pool_create(nblocks, 16, order)
    assert st_ == pa.PA_OK
    try:
        for op, seq, n in oplist:
            if op == "create":
                assert pa.pa_seq_create(pool, seq, n) == ref.seq_create(seq, n)
            elif op == "append":
                s1, slots1 = pa.pa_seq_append(pool, seq, n)
                s2, slots2 = ref.seq_append(seq, n)
                assert s1 == s2
                if s1 == pa.PA_OK and n > 0:
                    assert list(slots1) == slots2
            elif op == "release":
                assert pa.pa_seq_release(pool, seq) == ref.seq_release(seq)
            else:
                seqs = sorted(ref.tables)
                if seqs:
                    mb = max(1, max(len(t) for t in ref.tables.values()))
                    s1, t1, l1 = pa.pa_pack_batch(pool, seqs, mb)
                    t2, l2 = ref.pack(seqs, mb)
                    assert s1 == pa.PA_OK
                    assert t1.tolist() == t2 and l1.tolist() == l2
            assert _state(pool) == ref.free_list()
            assert pa.pa_pool_num_free(pool) == ref.num_free()
            assert pa.pa_pool_num_seqs(pool) == len(ref.tables)
            for s, t in ref.tables.items():
                st2, tab = pa.pa_seq_block_table(pool, s)
                assert st2 == pa.PA_OK and list(tab) == t
                st3, ln = pa.pa_seq_length(pool, s)
                assert ln == ref.lengths[s]
                if ref.lengths[s]:
                    st4, sl = pa.pa_seq_slots(pool, s, 0, ref.lengths[s])
                    assert list(sl) == ref.slots(s, 0, ref.lengths[s])
    finally:
        pa.pa_pool_destroy(pool)


def test_batch_append_matches_oracle_and_stops_at_failure():
    st_, pool = pa.pa_pool_create(5, 16, [4, 3, 2, 1, 0])
    ref = oa.BlockPool(5, 16, [4, 3, 2, 1, 0])
    try:
        for s, n in [(10, 16), (11, 5), (12, 32)]:
            assert pa.pa_seq_create(pool, s, n) == ref.seq_create(s, n) == pa.PA_OK
        # 10 crosses a boundary (takes 1), 11 does not, 12 needs one more: none left
        st2, done, slots = pa.pa_batch_append(pool, [11, 10, 12], 1)
        assert st2 == pa.PA_ERR_NO_BLOCKS and done == 2
        exp = [ref.seq_append(11, 1)[1], ref.seq_append(10, 1)[1]]
        assert slots[:2].tolist() == exp
        assert ref.seq_append(12, 1)[0] == oa.ERR_NO_BLOCKS
        assert _state(pool) == ref.free_list()
        assert pa.pa_seq_length(pool, 12) == (pa.PA_OK, 32)
    finally:
        pa.pa_pool_destroy(pool)


def test_error_paths_leave_state_unchanged():
    st_, pool = pa.pa_pool_create(3, 16, [2, 0, 1])
    assert st_ == pa.PA_OK
    try:
        assert pa.pa_seq_create(pool, 7, 40) == pa.PA_OK        # takes 2, 0, 1
        before = _state(pool)
        assert pa.pa_seq_append(pool, 7, 9)[0] == pa.PA_ERR_NO_BLOCKS
        assert "need 1 blocks, 0 free" in pa.pa_last_error()
        assert pa.pa_seq_length(pool, 7) == (pa.PA_OK, 40)
        assert _state(pool) == before
        assert pa.pa_seq_create(pool, 7, 1) == pa.PA_ERR_EXISTS
        assert pa.pa_seq_release(pool, 8) == pa.PA_ERR_UNKNOWN_SEQ
        assert pa.pa_seq_create(pool, 9, -1) == pa.PA_ERR_INVALID
        assert pa.pa_seq_slots(pool, 7, 39, 2)[0] == pa.PA_ERR_INVALID
        st2, _, _ = pa.pa_pack_batch(pool, [7], 2)              # table has 3 blocks
        assert st2 == pa.PA_ERR_INVALID
        assert pa.pa_seq_release(pool, 7) == pa.PA_OK
        assert _state(pool) == [2, 0, 1]
    finally:
        pa.pa_pool_destroy(pool)
    assert pa.pa_pool_create(3, 16, [0, 0, 1])[0] == pa.PA_ERR_INVALID
    assert pa.pa_pool_create(3, 0)[0] == pa.PA_ERR_INVALID
    assert pa.pa_pool_num_free(None) == -1


def test_validate_tables():
    t = np.array([[0, 1, -1], [2, -1, -1]], dtype=np.int32)
    assert pa.pa_validate_tables(t, [20, 16], 3, 16, 3) == pa.PA_OK
    assert pa.pa_validate_tables(t, [20, 17], 3, 16, 3) == pa.PA_ERR_INVALID   # needs entry [1][1]
    assert pa.pa_validate_tables(t, [49, 1], 3, 16, 3) == pa.PA_ERR_INVALID    # longer than 3 blocks
    assert pa.pa_validate_tables(t, [20, 16], 3, 16, 2) == pa.PA_ERR_INVALID   # block 2 out of pool


def test_argument_validation_of_kernel_entry_points_on_host():
    # invalid arguments are rejected before anything touches a device
    assert pa._pa._lib.pa_decode(None, None, 1, None, 1, None, None, 1, None, 4, 4, None,
                                 1, 64, 8, 128, 12, 100, 0.1, 1.0, 1.0, None, 0) == pa.PA_ERR_INVALID
    assert "block size" in pa.pa_last_error()
    # blocks of 8 or 32 tokens only on the matrix-core path: an fp32 call is
    # refused before any launch
    fake = 0x1000
    assert pa._pa._lib.pa_decode(None, fake, 0, fake, 0, fake, fake, 0, fake, 4, 4, fake,
                                 1, 4, 4, 64, 32, 100, 0.1, 1.0, 1.0, None, 0) == pa.PA_ERR_INVALID
    assert "matrix-core" in pa.pa_last_error()
    assert pa._pa._lib.pa_decode(None, None, 1, None, 1, None, None, 1, None, 4, 4, None,
                                 1, 64, 7, 128, 16, 100, 0.1, 1.0, 1.0, None, 0) == pa.PA_ERR_INVALID
    assert pa._pa._lib.pa_decode(None, None, 1, None, 1, None, None, 1, None, 4, 4, None,
                                 1, 64, 8, 96, 16, 100, 0.1, 1.0, 1.0, None, 0) == pa.PA_ERR_INVALID
    assert pa._pa._lib.pa_decode(None, None, 1, None, 1, None, None, 0, None, 4, 4, None,
                                 1, 64, 8, 128, 16, 100, 0.1, 1.0, 1.0, None, 0) == pa.PA_ERR_INVALID
    assert "dtypes" in pa.pa_last_error()
    # fp8 cache with a bad scale
    assert pa._pa._lib.pa_decode(None, None, 1, None, 1, None, None, 2, None, 4, 4, None,
                                 1, 64, 8, 128, 16, 100, 0.1, 0.0, 1.0, None, 0) == pa.PA_ERR_INVALID
    # the MFMA path needs its workspace (pointers are never dereferenced on this path)
    fake = 0x1000
    assert pa._pa._lib.pa_decode(None, fake, 1, fake, 1, fake, fake, 1, fake, 4, 4, fake,
                                 1, 64, 8, 128, 16, 100, 0.1, 1.0, 1.0, None, 0) == pa.PA_ERR_WORKSPACE
    assert pa.pa_decode_workspace_bytes(2, 64, 8, 128, 600) == 256 + 2 * 64 * 1 * 130 * 4
    assert pa.pa_decode_workspace_bytes(2, 64, 8, 128, 4097) == 256 + 2 * 64 * 3 * 130 * 4
    assert pa._pa._lib.pa_cache_write(None, None, None, 1, None, 4, None, None, 0, 4, 8, 128, 16,
                                      1.0, 1.0) == pa.PA_ERR_INVALID
    assert pa._pa._lib.pa_cache_write(None, fake, fake, 1, fake, 4, fake, fake, 2, 4, 8, 128, 16,
                                      -1.0, 1.0) == pa.PA_ERR_INVALID
    assert pa._pa._lib.pa_prefill_chunk(None, None, 1, None, 1, None, None, None, None, 1, None, 4,
                                        4, 1, 64, 8, 128, 8, 512, 512, 0.1, 1.0, 1.0, None,
                                        0) == pa.PA_ERR_INVALID


def test_stage_and_timing_argument_checks_on_host():
    # rejected before any HIP call
    fake = 0x1000
    assert pa._pa._lib.pa_stage(None, fake, fake, 0) == 0                # no-op
    assert pa._pa._lib.pa_stage(None, None, fake, 16) == pa.PA_ERR_INVALID
    assert pa._pa._lib.pa_stage(None, fake, fake, 6) == pa.PA_ERR_INVALID
    assert pa._pa._lib.pa_stage(None, fake + 2, fake, 8) == pa.PA_ERR_INVALID
    assert pa._pa._lib.pa_timing_enable(2, 0) == pa.PA_ERR_INVALID
    assert "every" in pa.pa_last_error()
    assert pa._pa._lib.pa_timing_enable(0, 1) == 0


def test_stage_cache_write_argument_checks_on_host():
    fake = 0x1000
    lib = pa._pa._lib
    # block size, dtypes, fp8 scale, slot range and alignment: rejected before any HIP call
    assert lib.pa_stage_cache_write(None, fake, fake, 64, 0, fake, fake, 1, 4, fake, fake, 1, 10,
                                    2, 64, 8, 1.0, 1.0) == pa.PA_ERR_INVALID
    assert lib.pa_stage_cache_write(None, fake, fake, 64, 0, fake, fake, 1, 4, fake, fake, 0, 10,
                                    2, 64, 16, 1.0, 1.0) == pa.PA_ERR_INVALID
    assert lib.pa_stage_cache_write(None, fake, fake, 64, 0, fake, fake, 1, 4, fake, fake, 2, 10,
                                    2, 64, 16, 0.0, 1.0) == pa.PA_ERR_INVALID
    assert lib.pa_stage_cache_write(None, fake, fake, 64, 52, fake, fake, 1, 4, fake, fake, 1, 10,
                                    2, 64, 16, 1.0, 1.0) == pa.PA_ERR_INVALID
    assert "do not fit" in pa.pa_last_error()
    assert lib.pa_stage_cache_write(None, fake, fake, 64, 6, fake, fake, 1, 4, fake, fake, 1, 10,
                                    2, 64, 16, 1.0, 1.0) == pa.PA_ERR_INVALID
    assert lib.pa_stage_cache_write(None, fake, fake, 0, 0, fake, fake, 1, 0, fake, fake, 1, 10,
                                    2, 64, 16, 1.0, 1.0) == 0          # nothing to do


def test_stage_decode_append_argument_checks_on_host():
    fake = 0x1000
    lib = pa._pa._lib
    # (stream, dst, src, bytes, slot_off, lens_off, k, v, new_dt, n, kc, vc, cache_dt,
    #  num_blocks, H_kv, D, bs, k_scale, v_scale, tables, max_blocks)
    ok = [None, fake, fake, 64, 0, 16, fake, fake, 1, 4, fake, fake, 1, 10, 2, 64, 16, 1.0, 1.0,
          fake, 8]

    def call(**kw):
        args = list(ok)
        names = ["stream", "dst", "src", "nbytes", "slot_off", "lens_off", "k", "v", "new_dt", "n",
                 "kc", "vc", "cache_dt", "num_blocks", "h_kv", "d", "bs", "k_scale", "v_scale",
                 "tables", "max_blocks"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.pa_stage_decode_append(*args)

    # all rejected before any HIP call
    assert call(lens_off=6) == pa.PA_ERR_INVALID                 # misaligned lengths
    assert call(lens_off=56) == pa.PA_ERR_INVALID                # 4 lengths do not fit 64 bytes
    assert "do not fit" in pa.pa_last_error()
    assert call(max_blocks=0) == pa.PA_ERR_INVALID
    assert call(tables=None) == pa.PA_ERR_INVALID
    assert "block_tables" in pa.pa_last_error()
    assert call(bs=8) == pa.PA_ERR_INVALID                       # as pa_stage_cache_write
    assert call(slot_off=52) == pa.PA_ERR_INVALID
    assert call(nbytes=0, n=0) == 0                              # nothing to do


def test_decode_append_argument_checks_on_host():
    fake = 0x1000
    lib = pa._pa._lib
    # (stream, slots, lens, n, k, v, new_dt, kc, vc, cache_dt, num_blocks, H_kv, D, bs,
    #  k_scale, v_scale, tables, max_blocks)
    ok = [None, fake, fake, 4, fake, fake, 1, fake, fake, 1, 10, 2, 64, 16, 1.0, 1.0, fake, 8]
    names = ["stream", "slots", "lens", "n", "k", "v", "new_dt", "kc", "vc", "cache_dt",
             "num_blocks", "h_kv", "d", "bs", "k_scale", "v_scale", "tables", "max_blocks"]

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.pa_decode_append(*args)

    # all rejected before any HIP call
    assert call(slots=None) == pa.PA_ERR_INVALID
    assert call(lens=None) == pa.PA_ERR_INVALID
    assert call(tables=None) == pa.PA_ERR_INVALID
    assert call(max_blocks=0) == pa.PA_ERR_INVALID
    assert call(bs=8) == pa.PA_ERR_INVALID                       # as pa_cache_write
    assert call(d=96) == pa.PA_ERR_INVALID
    assert call(n=0) == 0                                        # nothing to do


def test_decode_step_argument_checks_on_host():
    fake = 0x1000
    lib = pa._pa._lib
    names = ["stream", "dst", "src", "nbytes", "slot_off", "lens_off", "k", "v", "new_dt", "out",
             "out_dt", "q", "q_dt", "kc", "vc", "cache_dt", "tables", "max_blocks", "num_blocks",
             "S", "h_q", "h_kv", "d", "bs", "max_ctx", "sm_scale", "k_scale", "v_scale", "ws",
             "ws_bytes"]
    # 4 sequences, 16/2 heads, d 64, bf16 throughout; a workspace large enough
    need = pa.pa_decode_workspace_bytes(4, 16, 2, 64, 100)
    ok = [None, fake, fake, 32, 0, 16, fake, fake, 1, fake, 1, fake, 1, fake, fake, 1, fake, 8,
          10, 4, 16, 2, 64, 16, 100, 0.125, 1.0, 1.0, fake, need]

    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.pa_decode_step(*args)

    # all rejected before any HIP call
    assert call(bs=8) == pa.PA_ERR_INVALID
    assert call(S=2049) == pa.PA_ERR_INVALID                     # lengths kept in LDS
    assert call(h_q=48, h_kv=2) == pa.PA_ERR_INVALID             # 24 query heads per KV head
    assert call(d=96) == pa.PA_ERR_INVALID
    assert call(new_dt=0) == pa.PA_ERR_INVALID                   # f32 new K/V
    assert call(q_dt=0) == pa.PA_ERR_INVALID
    assert call(cache_dt=0) == pa.PA_ERR_INVALID
    assert call(cache_dt=2, k_scale=0.0) == pa.PA_ERR_INVALID    # fp8 scales
    assert call(sm_scale=float("nan")) == pa.PA_ERR_INVALID
    assert call(max_blocks=0) == pa.PA_ERR_INVALID
    assert call(max_ctx=0) == pa.PA_ERR_INVALID
    assert call(lens_off=6) == pa.PA_ERR_INVALID                 # misaligned
    assert call(lens_off=24) == pa.PA_ERR_INVALID                # 4 lengths do not fit 32 bytes
    assert "do not fit" in pa.pa_last_error()
    assert call(slot_off=20) == pa.PA_ERR_INVALID
    assert call(tables=None) == pa.PA_ERR_INVALID
    assert call(dst=None) == pa.PA_ERR_INVALID
    assert call(k=None) == pa.PA_ERR_INVALID
    assert call(ws=None) == pa.PA_ERR_WORKSPACE
    assert call(ws_bytes=need - 4) == pa.PA_ERR_WORKSPACE
    assert call(S=0, nbytes=0) == 0                              # nothing to do
    # the testing aid's limit is checked on the host
    assert lib.pa_decode_step_set_spin_limit(0) == pa.PA_ERR_INVALID
    assert lib.pa_decode_step_set_spin_limit(65536) == pa.PA_OK


def test_prefix_sharing_golden_trace_through_c_abi():
    g = json.load(open(os.path.join(GOLDEN, "prefix_sharing_trace.json")))
    st_, pool = pa.pa_pool_create(g["num_blocks"], g["block_size"], g["initial_free_order"])
    assert st_ == pa.PA_OK
    try:
        for step in g["steps"]:
            if step["op"] == "create":
                s = pa.pa_seq_create(pool, step["seq"], step["n"])
            elif step["op"] == "append":
                s, slots = pa.pa_seq_append(pool, step["seq"], step["n"])
                if "slots" in step:
                    assert list(slots) == step["slots"]
            elif step["op"] == "share":
                s, shared = pa.pa_seq_share(pool, step["seq"], step["src"], step["shared"],
                                            step["n"])
                if "shared_out" in step:
                    assert shared == step["shared_out"]
            else:
                s = pa.pa_seq_release(pool, step["seq"])
            assert s == step["status"], (step, pa.pa_last_error())
            assert _state(pool) == step["free"]
            if "table" in step:
                assert list(pa.pa_seq_block_table(pool, step["seq"])[1]) == step["table"]
            if "refs" in step:
                assert [pa.pa_pool_block_refs(pool, b)[1] for b in range(g["num_blocks"])] == \
                    step["refs"]
        assert pa.pa_pool_block_refs(pool, g["num_blocks"])[0] == pa.PA_ERR_INVALID
    finally:
        pa.pa_pool_destroy(pool)


def test_prefix_detection_golden_trace_through_c_abi():
    """tests/golden/prefix_detection_trace.json (hand-worked, ARTICLE 4.3)
    through the C ABI."""
    g = json.load(open(os.path.join(GOLDEN, "prefix_detection_trace.json")))
    st_, pool = pa.pa_pool_create(g["num_blocks"], g["block_size"], g["initial_free_order"])
    assert st_ == pa.PA_OK
    try:
        for step in g["steps"]:
            if step["op"] == "create_prefix":
                s, shared = pa.pa_seq_create_prefix(pool, step["seq"], step["tokens"])
                if s == pa.PA_OK and "shared_out" in step:
                    assert shared == step["shared_out"], step
            elif step["op"] == "register":
                s = pa.pa_seq_register_prefix(pool, step["seq"], step["tokens"])
            else:
                s = pa.pa_seq_release(pool, step["seq"])
            assert s == step["status"], (step, pa.pa_last_error())
            assert _state(pool) == step["free"], step
            assert pa.pa_pool_num_registered(pool) == step["registered"], step
            if "table" in step:
                assert list(pa.pa_seq_block_table(pool, step["seq"])[1]) == step["table"]
            if "refs" in step:
                assert [pa.pa_pool_block_refs(pool, b)[1] for b in range(g["num_blocks"])] == \
                    step["refs"]
    finally:
        pa.pa_pool_destroy(pool)


detect_ops = st.lists(st.tuples(st.sampled_from(["create", "register", "append", "release",
                                                 "match"]),
                                st.integers(0, 7), st.lists(st.integers(0, 1), max_size=40),
                                st.integers(0, 40)), max_size=80)


@settings(max_examples=300, deadline=None)
@given(detect_ops, st.integers(0, 40), st.randoms(use_true_random=False))
def test_prefix_detection_bit_exact_against_oracle(oplist, nblocks, rnd):
    """Random create-from-tokens / register / append / release / lookup
    sequences over a two-letter token alphabet (so that contents repeat and
    match):
    statuses, shared counts, tables, lengths, free list, reference counts
    and the number of registered blocks equal the oracle's after every
    operation."""
    order = list(range(nblocks))
    rnd.shuffle(order)
    ref = oa.BlockPool(nblocks, 4, order)
    st_, pool = pa.pa_pool_create(nblocks, 4, order)
    assert st_ == pa.PA_OK
    toks = {}   # token ids of every live sequence
    try:
        for op, seq, tokens, n in oplist:
            if op == "create":
                r1 = pa.pa_seq_create_prefix(pool, seq, tokens)
                r2 = ref.seq_create_prefix(seq, tokens)
                assert r1 == r2
                if r1[0] == pa.PA_OK:
                    toks[seq] = list(tokens)
            elif op == "register":
                t = toks.get(seq, [])[:n]
                assert pa.pa_seq_register_prefix(pool, seq, t) == ref.seq_register_prefix(seq, t)
            elif op == "match":
                st1, m1 = pa.pa_pool_match_prefix(pool, tokens)
                assert st1 == pa.PA_OK and m1 == ref.match_prefix(tokens)
            elif op == "append":
                s1, _ = pa.pa_seq_append(pool, seq, n % 9)
                s2, _ = ref.seq_append(seq, n % 9)
                assert s1 == s2
                if s1 == pa.PA_OK:
                    toks[seq] += [rnd.randint(0, 1) for _ in range(n % 9)]
            else:
                assert pa.pa_seq_release(pool, seq) == ref.seq_release(seq)
                toks.pop(seq, None)
            assert _state(pool) == ref.free_list()
            assert pa.pa_pool_num_registered(pool) == ref.num_registered()
            for b in range(nblocks):
                assert pa.pa_pool_block_refs(pool, b)[1] == ref.block_refs(b)
            for s, t in ref.tables.items():
                assert list(pa.pa_seq_block_table(pool, s)[1]) == t
                assert pa.pa_seq_length(pool, s)[1] == ref.lengths[s]
    finally:
        pa.pa_pool_destroy(pool)


share_ops = st.lists(st.tuples(st.sampled_from(["create", "append", "release", "share"]),
                               st.integers(0, 6), st.integers(0, 6), st.integers(0, 90),
                               st.integers(0, 90)), max_size=80)


@settings(max_examples=300, deadline=None)
@given(share_ops, st.integers(0, 48), st.randoms(use_true_random=False))
def test_prefix_sharing_bit_exact_against_oracle(oplist, nblocks, rnd):
    order = list(range(nblocks))
    rnd.shuffle(order)
    ref = oa.BlockPool(nblocks, 16, order)
    st_, pool = pa.pa_pool_create(nblocks, 16, order)
    assert st_ == pa.PA_OK
    try:
        for op, seq, src, n, shared in oplist:
            if op == "create":
                assert pa.pa_seq_create(pool, seq, n) == ref.seq_create(seq, n)
            elif op == "append":
                s1, slots1 = pa.pa_seq_append(pool, seq, n)
                s2, slots2 = ref.seq_append(seq, n)
                assert s1 == s2
                if s1 == pa.PA_OK and n > 0:
                    assert list(slots1) == slots2
            elif op == "share":
                assert pa.pa_seq_share(pool, seq, src, shared, n) == \
                    ref.seq_share(seq, src, shared, n)
            else:
                assert pa.pa_seq_release(pool, seq) == ref.seq_release(seq)
            assert _state(pool) == ref.free_list()
            for b in range(nblocks):
                assert pa.pa_pool_block_refs(pool, b)[1] == ref.block_refs(b)
            for s, t in ref.tables.items():
                assert list(pa.pa_seq_block_table(pool, s)[1]) == t
                assert pa.pa_seq_length(pool, s)[1] == ref.lengths[s]
    finally:
        pa.pa_pool_destroy(pool)


def test_prefix_retention_golden_trace_through_c_abi():
    """tests/golden/prefix_retention_trace.json (hand-worked) through the C
    allocator: statuses, shared and matched counts, tables, free list,
    registered and retained counts, reference counts."""
    g = json.load(open(os.path.join(GOLDEN, "prefix_retention_trace.json")))
    st_, pool = pa.pa_pool_create(g["num_blocks"], g["block_size"], g["initial_free_order"])
    assert st_ == pa.PA_OK
    try:
        for i, step in enumerate(g["steps"]):
            op = step["op"]
            res = {}
            if op == "retention":
                res["status"] = pa.pa_pool_set_prefix_retention(pool, step["on"])
            elif op == "create_prefix":
                res["status"], res["shared_out"] = pa.pa_seq_create_prefix(pool, step["seq"],
                                                                           step["tokens"])
            elif op == "register":
                res["status"] = pa.pa_seq_register_prefix(pool, step["seq"], step["tokens"])
            elif op == "release":
                res["status"] = pa.pa_seq_release(pool, step["seq"])
            elif op == "create":
                res["status"] = pa.pa_seq_create(pool, step["seq"], step["n"])
            else:
                res["status"], res["matched"], res["matched_retained"] = \
                    pa.pa_pool_match_prefix(pool, step["tokens"], with_retained=True)
            res["free"] = _state(pool)
            res["registered"] = pa.pa_pool_num_registered(pool)
            res["retained"] = pa.pa_pool_num_retained(pool)
            if "table" in step:
                res["table"] = list(pa.pa_seq_block_table(pool, step["seq"])[1])
            if "refs" in step:
                res["refs"] = [pa.pa_pool_block_refs(pool, b)[1] for b in range(g["num_blocks"])]
            for k, v in step.items():
                if k in res and not (k == "shared_out" and res["status"] != pa.PA_OK):
                    assert res[k] == v, (i, op, k, res[k], v)
    finally:
        pa.pa_pool_destroy(pool)


retain_ops = st.lists(st.tuples(st.sampled_from(["create", "register", "append", "release",
                                                 "match", "plain", "retain_on", "retain_off"]),
                                st.integers(0, 7), st.lists(st.integers(0, 1), max_size=40),
                                st.integers(0, 40)), max_size=80)


@settings(max_examples=300, deadline=None)
@given(retain_ops, st.integers(0, 40), st.randoms(use_true_random=False))
def test_prefix_retention_bit_exact_against_oracle(oplist, nblocks, rnd):
    """Random sequences of the detection operations, plain creates and
    retention switched on and off, over a two-letter token alphabet: every
    status, count, table, the free list (retained blocks after it) and the
    reference counts equal the oracle's after every operation."""
    order = list(range(nblocks))
    rnd.shuffle(order)
    ref = oa.BlockPool(nblocks, 4, order)
    st_, pool = pa.pa_pool_create(nblocks, 4, order)
    assert st_ == pa.PA_OK
    ref.set_prefix_retention(True)
    assert pa.pa_pool_set_prefix_retention(pool, True) == pa.PA_OK
    toks = {}
    try:
        for op, seq, tokens, n in oplist:
            if op == "create":
                r1 = pa.pa_seq_create_prefix(pool, seq, tokens)
                assert r1 == ref.seq_create_prefix(seq, tokens)
                if r1[0] == pa.PA_OK:
                    toks[seq] = list(tokens)
            elif op == "plain":
                s1 = pa.pa_seq_create(pool, seq, n)
                assert s1 == ref.seq_create(seq, n)
                if s1 == pa.PA_OK:
                    toks[seq] = [rnd.randint(0, 1) for _ in range(n)]
            elif op == "register":
                t = toks.get(seq, [])[:n]
                assert pa.pa_seq_register_prefix(pool, seq, t) == ref.seq_register_prefix(seq, t)
            elif op == "match":
                st1, m1, r1 = pa.pa_pool_match_prefix(pool, tokens, with_retained=True)
                assert st1 == pa.PA_OK and (m1, r1) == ref.match_prefix(tokens, with_retained=True)
            elif op == "append":
                s1, _ = pa.pa_seq_append(pool, seq, n % 9)
                assert s1 == ref.seq_append(seq, n % 9)[0]
                if s1 == pa.PA_OK:
                    toks[seq] += [rnd.randint(0, 1) for _ in range(n % 9)]
            elif op == "release":
                assert pa.pa_seq_release(pool, seq) == ref.seq_release(seq)
                toks.pop(seq, None)
            else:
                on = op == "retain_on"
                assert pa.pa_pool_set_prefix_retention(pool, on) == ref.set_prefix_retention(on)
            assert _state(pool) == ref.free_list()
            assert pa.pa_pool_num_free(pool) == ref.num_free()
            assert pa.pa_pool_num_registered(pool) == ref.num_registered()
            assert pa.pa_pool_num_retained(pool) == ref.num_retained()
            for b in range(nblocks):
                assert pa.pa_pool_block_refs(pool, b)[1] == ref.block_refs(b)
            for s, t in ref.tables.items():
                assert list(pa.pa_seq_block_table(pool, s)[1]) == t
    finally:
        pa.pa_pool_destroy(pool)


class _CPoolView:
    """The C allocator behind the interface tests/prefix_truth.py drives."""

    def __init__(self, num_blocks, block_size):
        st_, self.pool = pa.pa_pool_create(num_blocks, block_size, None)
        assert st_ == pa.PA_OK
        self.block_size = block_size

    def seq_create_prefix(self, seq, tokens):
        return pa.pa_seq_create_prefix(self.pool, seq, tokens)

    def block_table(self, seq):
        return list(pa.pa_seq_block_table(self.pool, seq)[1])

    def free_list(self):
        return _state(self.pool)

    def seq_append(self, seq, n):
        return pa.pa_seq_append(self.pool, seq, n)

    def seq_register_prefix(self, seq, tokens):
        return pa.pa_seq_register_prefix(self.pool, seq, tokens)

    def seq_release(self, seq):
        return pa.pa_seq_release(self.pool, seq)

    def set_prefix_retention(self, on):
        assert pa.pa_pool_set_prefix_retention(self.pool, on) == pa.PA_OK


def test_prefix_blocks_hold_their_own_prefix_through_c_abi():
    """The oracle's 6000 seeded random runs (prompts, appends, registrations,
    releases, retention switched on and off, pools small enough that retained
    blocks are evicted all the time) through the C allocator: no sequence is
    ever handed a block computed under a different prefix."""
    for ops, nblocks in seeded_cases():
        view = _CPoolView(nblocks, 2)
        try:
            run_with_truth(view, ops, check_index=False)
        finally:
            pa.pa_pool_destroy(view.pool)
