"""GPU parity: pa_cache_write (bit-exact) and pa_decode (tolerance) against
the oracle, through the C ABI."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import codecs
from tests.parity import assert_close, filled, hip_decode_run, oracle_decode_run, out_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _edge_workload(lengths, h_q, h_kv, d, dtype, cache_dtype, seed, extra_blocks=7):
    lengths = np.asarray(lengths, dtype=np.int64)
    return workloads.decode_workload(
        f"edge-{dtype}-{cache_dtype}-{h_q}q{h_kv}kv-d{d}", seed, lambda rng: lengths,
        h_q, h_kv, d, dtype, cache_dtype,
        lambda L: workloads.blocks_needed(L) + extra_blocks,
        q_dtype="bf16" if cache_dtype == "fp8" else dtype)


def _check_full(w, what):
    say(f"[decode parity] {what}: {w.name} S={w.num_seqs} maxL={int(w.lengths.max())}")
    hip = hip_decode_run(w, DEV)
    ref = oracle_decode_run(w)
    # allocator state, slots and cache bytes bit-exact
    assert np.array_equal(hip["tables"], ref["tables"])
    assert np.array_equal(hip["lens"], ref["lens"])
    assert np.array_equal(hip["slots"], ref["slots"])
    kc = hip["kv"].k.cpu().numpy().view(ref["kc"].dtype) if w.cache_dtype != "bf16" else \
        hip["kv"].k.cpu().view(torch.int16).numpy().view(np.uint16)
    vc = hip["kv"].v.cpu().numpy().view(ref["vc"].dtype) if w.cache_dtype != "bf16" else \
        hip["kv"].v.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kc, ref["kc"]), "K cache bytes differ"
    assert np.array_equal(vc, ref["vc"]), "V cache bytes differ"
    got = out_to_f64(hip["outs"][0], w.q_dtype)
    err = assert_close(got, ref["out"], w.cache_dtype, what)
    say(f"    max|d| = {err:.3g}")
    hip["kv"].close()


@pytest.mark.parametrize("h_q,h_kv", [(16, 2), (64, 8)])
def test_rising_scores_bf16(h_q, h_kv):
    """Scores that climb about 8 powers of two per 64 keys: every step of a
    context outweighs the running maximum, so each wave keeps raising its
    reference, and the waves' and chunks' states merge across far apart
    maxima (the 2500-token context spans two work items)."""
    lengths = np.array([1, 63, 64, 700, 2500, 130], dtype=np.int64)
    w = workloads.decode_workload(
        f"rising-{h_q}q{h_kv}kv", 913 + h_q, lambda rng: lengths, h_q, h_kv, 128, "bf16", "bf16",
        lambda L: workloads.blocks_needed(L) + 7, score_ramp=8.0)
    _check_full(w, "scores rising 8 per 64 keys")


def test_tiny_decode_f32():
    _check_full(workloads.tiny_decode(), "tiny fp32")


@pytest.mark.parametrize("h_q,h_kv,d", [(64, 8, 128), (16, 2, 64), (8, 8, 128), (32, 2, 128),
                                        (64, 2, 128)])
def test_edge_lengths_bf16(h_q, h_kv, d):
    lengths = [1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1000, 4097]
    _check_full(_edge_workload(lengths, h_q, h_kv, d, "bf16", "bf16", seed=100 + h_q + d),
                f"edge bf16 {h_q}/{h_kv} d{d}")


@pytest.mark.parametrize("h_q,h_kv,d", [(64, 8, 128), (16, 4, 64)])
def test_edge_lengths_fp8(h_q, h_kv, d):
    lengths = [1, 2, 16, 17, 33, 256, 257, 700, 2049]
    _check_full(_edge_workload(lengths, h_q, h_kv, d, "bf16", "fp8", seed=200 + h_q + d),
                f"edge fp8 {h_q}/{h_kv} d{d}")


@pytest.mark.parametrize("S,long_lengths", [
    # 34 x 8 x 9000 ~ 2.4M KV rows in the launch bound: 4096-token work items
    (34, [2047, 2048, 2049, 4095, 4096, 4097, 8192, 9000]),
    # 34 x 8 x 16385 ~ 4.5M: 8192-token work items
    (34, [4097, 8191, 8192, 8193, 16384, 16385]),
])
def test_large_work_items(S, long_lengths):
    """Launches whose size selects the longer work items: contexts that end
    on and beside the item boundaries (one, two and three items, merged)
    beside short ones; the oracle runs on the long sequences and two short
    ones."""
    rng = np.random.default_rng(500 + max(long_lengths))
    short = rng.integers(1, 300, S - len(long_lengths))
    lengths = np.concatenate([long_lengths, short])
    w = _edge_workload(lengths, 64, 8, 128, "bf16", "bf16", seed=S + max(long_lengths))
    say(f"[decode parity] large items: {w.name} S={w.num_seqs} maxL={int(w.lengths.max())}")
    hip = hip_decode_run(w, DEV)
    seqs = list(range(len(long_lengths))) + [len(long_lengths), S - 1]
    ref = oracle_decode_run(w, seqs=seqs)
    assert np.array_equal(hip["tables"], ref["tables"])
    assert np.array_equal(hip["slots"], ref["slots"])
    got = out_to_f64(hip["outs"][0], "bf16")
    err = assert_close(got[seqs], ref["out"][seqs], "bf16", "large items")
    say(f"    max|d| = {err:.3g}")
    hip["kv"].close()


def test_many_sequences_two_launches():
    """More sequences than one launch takes (4096): the launcher splits the
    batch; with more than 512 sequences the partial items keep index order.
    Oracle on sampled sequences of both launches."""
    rng = np.random.default_rng(600)
    lengths = rng.integers(1, 40, 5000)
    w = _edge_workload(lengths, 8, 2, 64, "bf16", "bf16", seed=601, extra_blocks=3)
    say(f"[decode parity] many sequences: {w.name} S={w.num_seqs}")
    hip = hip_decode_run(w, DEV)
    seqs = [0, 1, 511, 512, 4095, 4096, 4097, 4999]
    ref = oracle_decode_run(w, seqs=seqs)
    assert np.array_equal(hip["tables"], ref["tables"])
    assert np.array_equal(hip["slots"], ref["slots"])
    got = out_to_f64(hip["outs"][0], "bf16")
    err = assert_close(got[seqs], ref["out"][seqs], "bf16", "many sequences")
    say(f"    max|d| = {err:.3g}")
    hip["kv"].close()


def test_edge_lengths_f32_gqa():
    _check_full(_edge_workload([1, 16, 17, 100, 300], 8, 2, 64, "f32", "f32", seed=300),
                "edge f32 8/2 d64")


def test_decode_70b_full():
    """The 70B-shaped decode workload at full size: every output."""
    _check_full(workloads.decode_70b(), "70b-shaped full")


def test_fp8_long_context_sampled():
    """64 x 8192 fp8 workload: full device run, oracle on six sequences
    spread over the batch (cache bytes compared on their blocks); the
    oracle's fp8 encode takes about 7 s per sequence, all 64 about 450 s."""
    w = workloads.decode_fp8_long()
    say(f"[decode parity] fp8 long: {w.name}")
    hip = hip_decode_run(w, DEV)
    seqs = [0, 17, 31, 32, 48, 63]
    ref = oracle_decode_run(w, seqs=seqs)
    assert np.array_equal(hip["tables"], ref["tables"])
    assert np.array_equal(hip["slots"], ref["slots"])
    kc = hip["kv"].k.cpu().numpy()
    vc = hip["kv"].v.cpu().numpy()
    for s in seqs:
        blocks = ref["tables"][s][ref["tables"][s] >= 0]
        assert np.array_equal(kc[blocks], ref["kc"][blocks])
        assert np.array_equal(vc[blocks], ref["vc"][blocks])
    got = out_to_f64(hip["outs"][0], "bf16")
    err = assert_close(got[seqs], ref["out"][seqs], "fp8", "fp8 long")
    say(f"    max|d| = {err:.3g}")
    hip["kv"].close()


def test_block_permutation_and_repeat_are_bit_identical():
    w = _edge_workload([5, 16, 40, 300, 1025], 64, 8, 128, "bf16", "bf16", seed=400, extra_blocks=40)
    a = hip_decode_run(w, DEV, reps=2)
    rng = np.random.default_rng(401)
    b = hip_decode_run(w, DEV, free_order=rng.permutation(w.num_blocks).astype(np.int32))
    assert not np.array_equal(a["tables"], b["tables"])
    assert np.array_equal(a["outs"][0], a["outs"][1])      # run-to-run determinism
    assert np.array_equal(a["outs"][0], b["outs"][0])      # physical placement is invisible
    a["kv"].close()
    b["kv"].close()


def test_fp8_codes_decode_exactly():
    """One-token contexts: the output is the single value row, so every
    finite e4m3fn code must come out as its exact value (bf16 holds every
    e4m3fn value exactly)."""
    import paged_kv_cache_host_amd as pa
    from paged_kv_cache_host_amd.engine import PagedKV, decode_workspace
    h_q = h_kv = 2
    d = 128
    kv = PagedKV(4, h_kv, d, "fp8", DEV, None, 1.0, 1.0)
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    codes = np.where(np.isnan(codecs.E4M3_TABLE[codes]), 0x38, codes).astype(np.uint8)  # 0x38 = 1.0
    assert kv.create(0, 1) == 0
    v = torch.zeros((4, h_kv, d, 16), dtype=torch.uint8)      # V layout [b][h][D][16]
    st, table = pa.pa_seq_block_table(kv.pool, 0)
    v[int(table[0]), :, :, 0] = torch.from_numpy(codes)
    kv.v.copy_(v.to(DEV))
    kv.k.fill_(0x38)
    tables, lens = kv.pack([0])
    q = torch.ones((1, h_q, d), dtype=torch.bfloat16, device=DEV)
    out = filled(q.shape, q.dtype, DEV)
    ws = decode_workspace(1, h_q, h_kv, d, 1, DEV)
    kv.decode(out, q, torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV), 1,
              1.0 / math.sqrt(d), ws)
    got = out.float().cpu().numpy()[0]
    assert np.array_equal(got.astype(np.float64), codecs.E4M3_TABLE[codes])
    kv.close()


@pytest.mark.parametrize("bs,cache_dt", [(8, "bf16"), (32, "bf16"), (8, "fp8"), (32, "fp8")])
def test_block_sizes_8_and_32(bs, cache_dt):
    """pa_decode over caches of 8- and 32-token blocks (ARTICLE 4.1): the C
    allocator's tables for that block size equal the oracle's; the cache is
    scattered here by layout alone (its bytes equal the oracle's scatter);
    outputs within tolerance of the oracle.  Contexts around both block
    sizes and spanning two work items."""
    from oracle import allocator as oa
    from oracle import attention as oat
    from oracle import cache as oc
    import paged_kv_cache_host_amd._pa as pa
    rng = np.random.default_rng(1700 + bs + len(cache_dt))
    lengths = [1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 100, 700, 2500]
    S, h_q, h_kv, d = len(lengths), 16, 2, 128
    nb = sum(-(-L // bs) for L in lengths) + 7
    order = rng.permutation(nb).astype(np.int32)
    ntok = sum(lengths)
    if cache_dt == "bf16":
        k_raw = workloads.normal_raw(rng, (ntok, h_kv, d), "bf16")
        v_raw = workloads.normal_raw(rng, (ntok, h_kv, d), "bf16")
        ks = vs = 1.0
    else:   # e4m3fn codes, NaN codes (0x7F, 0xFF) excluded
        k_raw = rng.integers(0, 0x7F, size=(ntok, h_kv, d)).astype(np.uint8) | \
            (rng.integers(0, 2, size=(ntok, h_kv, d)).astype(np.uint8) << 7)
        v_raw = rng.integers(0, 0x7F, size=(ntok, h_kv, d)).astype(np.uint8) | \
            (rng.integers(0, 2, size=(ntok, h_kv, d)).astype(np.uint8) << 7)
        ks, vs = 0.01, 0.02
    q_raw = workloads.normal_raw(rng, (S, h_q, d), "bf16")
    # host side: the C allocator with this block size
    st_, pool = pa.pa_pool_create(nb, bs, order)
    assert st_ == pa.PA_OK
    try:
        slots = []
        for s, L in enumerate(lengths):
            assert pa.pa_seq_create(pool, s, L) == pa.PA_OK
            st_, sl = pa.pa_seq_slots(pool, s, 0, L)
            assert st_ == pa.PA_OK
            slots.append(np.asarray(sl, dtype=np.int64))
        mb = max(-(-L // bs) for L in lengths)
        st_, tables, lens = pa.pa_pack_batch(pool, np.arange(S), mb)
        assert st_ == pa.PA_OK
    finally:
        pa.pa_pool_destroy(pool)
    slots = np.concatenate(slots)
    # oracle allocator: same tables and slots
    opool = oa.BlockPool(nb, bs, order.tolist())
    for s, L in enumerate(lengths):
        assert opool.seq_create(s, L) == 0
    o_slots = np.concatenate([np.asarray(opool.slots(s, 0, L)) for s, L in enumerate(lengths)])
    assert np.array_equal(o_slots, slots)
    for s in range(S):
        t = opool.block_table(s)
        assert list(tables[s, :len(t)]) == list(t)
    # the device cache, scattered by layout only
    x = 8 if cache_dt == "bf16" else 16
    sdt = np.uint16 if cache_dt == "bf16" else np.uint8
    kc = np.zeros((nb, h_kv, d // x, bs, x), dtype=sdt)
    vc = np.zeros((nb, h_kv, d, bs), dtype=sdt)
    kc[slots // bs, :, :, slots % bs, :] = k_raw.reshape(ntok, h_kv, d // x, x)
    vc[slots // bs, :, :, slots % bs] = v_raw
    okc, ovc = oc.new_cache(nb, h_kv, bs, d, cache_dt)
    oc.cache_write(okc, ovc, k_raw, v_raw, slots, cache_dt, cache_dt)
    assert np.array_equal(okc, kc) and np.array_equal(ovc, vc)
    sm = float(np.float32(1.0) / np.float32(np.sqrt(d)))
    ref = oat.decode(codecs.decode(q_raw, "bf16"), okc, ovc, tables, lens, h_kv, sm, cache_dt,
                     ks, vs)
    k_d = torch.from_numpy(kc.view(np.int16) if cache_dt == "bf16" else kc).to(DEV)
    v_d = torch.from_numpy(vc.view(np.int16) if cache_dt == "bf16" else vc).to(DEV)
    if cache_dt == "bf16":
        k_d, v_d = k_d.view(torch.bfloat16), v_d.view(torch.bfloat16)
    else:
        k_d, v_d = k_d.view(torch.float8_e4m3fn), v_d.view(torch.float8_e4m3fn)
    q_d = torch.from_numpy(q_raw.view(np.int16)).to(DEV).view(torch.bfloat16)
    out = filled((S, h_q, d), torch.bfloat16, DEV)
    ws = torch.zeros(pa.pa_decode_workspace_bytes(S, h_q, h_kv, d, max(lengths)),
                     dtype=torch.uint8, device=DEV)
    say(f"[decode bs={bs}] {cache_dt} S={S} maxL={max(lengths)} pool={nb}")
    assert pa.pa_decode(None, out, q_d, k_d, v_d, torch.from_numpy(tables).to(DEV),
                        torch.from_numpy(lens).to(DEV), nb, h_kv, max(lengths), sm, ks, vs, ws,
                        bs=bs) == 0
    torch.cuda.synchronize()
    got = codecs.decode(out.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    err = assert_close(got, ref, cache_dt, f"bs={bs} {cache_dt}")
    say(f"    max|d| = {err:.3g}")


@pytest.mark.parametrize("bs", [8, 32])
@pytest.mark.parametrize("new_dt,cache_dt,d", [("f32", "f32", 64), ("bf16", "bf16", 128),
                                               ("bf16", "fp8", 128)])
def test_cache_write_block_sizes_8_and_32(bs, new_dt, cache_dt, d):
    """pa_cache_write into caches of 8- and 32-token blocks: slots from the C
    allocator with that block size (equal to the oracle allocator's), cache
    bytes bit-exact against the oracle's scatter (fp8: quantised with the
    per-tensor scales), every other byte of the cache left as it was."""
    from oracle import allocator as oa
    from oracle import cache as oc
    import paged_kv_cache_host_amd._pa as pa
    rng = np.random.default_rng(2500 + bs + d + len(cache_dt))
    lengths = [1, 7, 8, 9, 31, 33, 100, 257]
    h_kv = 2
    nb = sum(-(-L // bs) for L in lengths) + 5
    order = rng.permutation(nb).astype(np.int32)
    st_, pool = pa.pa_pool_create(nb, bs, order)
    assert st_ == pa.PA_OK
    try:
        slots = []
        for s, L in enumerate(lengths):
            assert pa.pa_seq_create(pool, s, L) == pa.PA_OK
            slots.append(np.asarray(pa.pa_seq_slots(pool, s, 0, L)[1], dtype=np.int64))
    finally:
        pa.pa_pool_destroy(pool)
    slots = np.concatenate(slots)
    opool = oa.BlockPool(nb, bs, order.tolist())
    for s, L in enumerate(lengths):
        assert opool.seq_create(s, L) == oa.OK
    assert np.array_equal(np.concatenate([opool.slots(s, 0, L) for s, L in enumerate(lengths)]),
                          slots)
    n = len(slots)
    k_raw = workloads.normal_raw(rng, (n, h_kv, d), new_dt)
    v_raw = workloads.normal_raw(rng, (n, h_kv, d), new_dt)
    ks, vs = (0.05, 0.03) if cache_dt == "fp8" else (1.0, 1.0)
    okc, ovc = oc.new_cache(nb, h_kv, bs, d, cache_dt)
    oc.cache_write(okc, ovc, k_raw, v_raw, slots, new_dt, cache_dt, ks, vs)
    x = 16 // {"f32": 4, "bf16": 2, "fp8": 1}[cache_dt]
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[cache_dt]
    raw_np = {"f32": np.int32, "bf16": np.int16, "fp8": np.uint8}[cache_dt]
    raw_t = {"f32": torch.int32, "bf16": torch.int16, "fp8": torch.uint8}[cache_dt]
    # the cache starts as a recognisable byte pattern, so stray writes show
    pattern = 0x3C if cache_dt == "fp8" else (0x3C3C if cache_dt == "bf16" else 0x3C3C3C3C)
    kc = torch.full(okc.shape, pattern, dtype=raw_t, device=DEV).view(tdt)
    vc = torch.full(ovc.shape, pattern, dtype=raw_t, device=DEV).view(tdt)

    def dev_raw(a):
        if new_dt == "f32":
            return torch.from_numpy(a.view(np.float32)).to(DEV)
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    say(f"[cache_write bs={bs}] {new_dt}->{cache_dt} d={d} n={n} pool={nb}")
    assert pa.pa_cache_write(None, dev_raw(k_raw), dev_raw(v_raw),
                             torch.from_numpy(slots.astype(np.int32)).to(DEV), kc, vc, nb, h_kv,
                             d, bs=bs, k_scale=ks, v_scale=vs) == pa.PA_OK
    torch.cuda.synchronize()
    got_k = kc.view(raw_t).cpu().numpy().view(okc.dtype)
    got_v = vc.view(raw_t).cpu().numpy().view(ovc.dtype)
    fill = np.array([pattern], dtype=raw_np).view(okc.dtype)[0]
    held = np.zeros(nb * bs, dtype=bool)
    held[slots] = True
    k_mask = held.reshape(nb, 1, 1, bs, 1).repeat(h_kv, 1).repeat(d // x, 2).repeat(x, 4)
    v_mask = held.reshape(nb, 1, 1, bs).repeat(h_kv, 1).repeat(d, 2)
    assert np.array_equal(got_k[k_mask], okc[k_mask])
    assert np.array_equal(got_v[v_mask], ovc[v_mask])
    assert np.all(got_k[~k_mask] == fill) and np.all(got_v[~v_mask] == fill)
