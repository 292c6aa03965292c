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
from tests.parity import assert_close, hip_decode_run, oracle_decode_run, out_to_f64

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
    """64 x 8192 fp8 workload: full device run, oracle on sampled sequences
    (cache bytes compared on those sequences' blocks)."""
    w = workloads.decode_fp8_long()
    say(f"[decode parity] fp8 long: {w.name}")
    hip = hip_decode_run(w, DEV)
    seqs = [0, 17, 63]
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
    out = torch.empty_like(q)
    ws = decode_workspace(1, h_q, h_kv, d, 1, DEV)
    kv.decode(out, q, torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV), 1,
              1.0 / math.sqrt(d), ws)
    got = out.float().cpu().numpy()[0]
    assert np.array_equal(got.astype(np.float64), codecs.E4M3_TABLE[codes])
    kv.close()
