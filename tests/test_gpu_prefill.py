"""GPU parity: pa_prefill_chunk (causal slices against the paged prefix)
against the oracle, through the C ABI."""
import sys

import numpy as np
import pytest

import workloads
from tests.parity import assert_close, filled, out_to_f64
from tests.prefill_parity import hip_prefill_run, oracle_prefill_run

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(w, what):
    say(f"[prefill parity] {what}: {w.name} slices={w.slices}")
    hip = hip_prefill_run(w, "cuda")
    ref = oracle_prefill_run(w)
    err = assert_close(out_to_f64(hip["out"], w.q_dtype), ref["out"], w.cache_dtype, what)
    say(f"    max|d| = {err:.3g}")
    hip["kv"].close()


@pytest.mark.parametrize("h_q,h_kv,d", [(64, 8, 128), (16, 2, 64), (8, 8, 128)])
def test_slices_one_prompt_bf16(h_q, h_kv, d):
    w = workloads.prefill_workload("one-prompt", 500 + h_q + d, prompt_len=333,
                                   chunks=[128, 100, 1, 64, 40], h_q=h_q, h_kv=h_kv, d=d)
    _check(w, f"bf16 {h_q}/{h_kv} d{d}")


def test_slices_several_prompts_bf16():
    w = workloads.prefill_workload("multi-prompt", 510, prompts=[700, 50, 1, 300],
                                   slices=[(0, 512, 188), (1, 0, 50), (2, 0, 1), (3, 256, 44),
                                           (0, 0, 130)])
    _check(w, "bf16 several prompts")


def test_slices_fp8():
    w = workloads.prefill_workload("fp8", 520, prompt_len=290, chunks=[130, 97, 63],
                                   cache_dtype="fp8")
    _check(w, "fp8 cache")


@pytest.mark.parametrize("prompt,chunks,h_q,h_kv,ramp",
                         [(700, [300, 400], 16, 2, 10.0), (2900, [2600, 300], 64, 8, 3.0)])
def test_slices_rising_scores(prompt, chunks, h_q, h_kv, ramp):
    """Scores that climb by `ramp` powers of two per 64 keys: each new tile
    outweighs the softmax reference taken so far, so the kernel keeps
    raising it (and rescaling what it has accumulated); the second case also
    splits the key range of the last slice."""
    w = workloads.prefill_workload("rising", 560 + prompt, prompt_len=prompt, chunks=chunks,
                                   h_q=h_q, h_kv=h_kv, score_ramp=ramp)
    _check(w, f"scores rising {ramp} per tile")


def test_slices_f32():
    w = workloads.prefill_workload("f32", 530, prompt_len=150, chunks=[64, 86], h_q=4, h_kv=4, d=64,
                                   dtype="f32", cache_dtype="f32")
    _check(w, "f32")


# Work decompositions of the matrix-core kernel: query heads per KV head of
# 1 (eight 32-position sub-tiles per work-group), 3 (two sub-tiles, six live
# waves), 4, 8 and 16 (two head groups); head dims 64 and 128.
@pytest.mark.parametrize("h_q,h_kv,d", [(32, 8, 128), (12, 4, 64), (32, 2, 128), (4, 4, 64)])
def test_slices_head_groupings(h_q, h_kv, d):
    w = workloads.prefill_workload("groups", 540 + h_q + d, prompt_len=420,
                                   chunks=[200, 33, 150, 37], h_q=h_q, h_kv=h_kv, d=d)
    _check(w, f"bf16 {h_q}/{h_kv} d{d}")


# Long prefixes with few query rows: the key range is split over several
# work-groups and the partial softmax states merged (2, 3 and 4 ranges).
@pytest.mark.parametrize("prompt,start,n,cache", [(2900, 2600, 300, "bf16"),
                                                   (5000, 4900, 100, "bf16"),
                                                   (3100, 2900, 200, "fp8")])
def test_slices_split_key_range(prompt, start, n, cache):
    w = workloads.prefill_workload("split", 560 + n, prompts=[prompt], slices=[(0, start, n)],
                                   cache_dtype=cache)
    _check(w, f"{cache} split prefix {start}+{n}")


def test_slices_split_several_prompts():
    w = workloads.prefill_workload("split-multi", 575, prompts=[2200, 1300, 2100],
                                   slices=[(0, 2100, 100), (1, 1280, 20), (2, 1000, 64)])
    _check(w, "bf16 split, several prompts")


def test_slices_single_token_and_block_edges():
    # slices of 1, 15, 16, 17 and 64 tokens starting on and off block edges
    w = workloads.prefill_workload("edges", 590, prompt_len=300,
                                   chunks=[1, 15, 16, 17, 64, 63, 65, 1, 48])
    _check(w, "bf16 block edges")


def _mixed_prefix_run(chunks, sample):
    """The 32768-token prompt of the mixed chunked-prefill workload, each
    listed 512-token slice launched alone exactly as the benchmark does;
    ``sample(c)`` gives the rows compared against the oracle (None = all)."""
    import torch

    from oracle import allocator as oa
    from oracle import attention as oat
    from oracle import cache as oc
    from oracle import codecs
    from paged_kv_cache_host_amd.engine import PagedKV, prefill_workspace, to_device_raw, to_host_raw

    w = workloads.mixed_prefill()
    dev = "cuda"
    P, C = w.prompt_len, w.chunk
    kv = PagedKV(w.num_blocks, w.h_kv, w.d, "bf16", dev, w.free_order)
    assert kv.create(0, P) == 0
    slots = kv.slots(0, 0, P).astype(np.int32)
    kv.write(to_device_raw(w.prompt_k, "bf16", dev), to_device_raw(w.prompt_v, "bf16", dev),
             torch.from_numpy(slots).to(dev))
    tables, _ = kv.pack([0], P // 16)
    t_d = torch.from_numpy(tables).to(dev)

    pool = oa.BlockPool(w.num_blocks, 16, w.free_order.tolist())
    assert pool.seq_create(0, P) == oa.OK
    assert np.array_equal(np.asarray(pool.block_table(0)), tables[0]), "tables differ"
    kc, vc = oc.new_cache(w.num_blocks, w.h_kv, 16, w.d, "bf16")
    oc.cache_write(kc, vc, w.prompt_k, w.prompt_v, pool.slots(0, 0, P), "bf16", "bf16")

    for c in chunks:
        P0 = c * C
        say(f"[prefill parity] mixed-prefill chunk {c} (prefix {P0})")
        q = to_device_raw(w.prompt_q[P0:P0 + C], "bf16", dev)
        out = filled((C, w.h_q, w.d), torch.bfloat16, dev)
        cu = torch.tensor([0, C], dtype=torch.int32, device=dev)
        st = torch.tensor([P0], dtype=torch.int32, device=dev)
        ws = prefill_workspace(1, C, w.h_q, w.h_kv, w.d, P0 + C, dev)
        kv.prefill(out, q, cu, st, t_d, C, P0 + C, w.sm_scale, ws)
        torch.cuda.synchronize()
        got = out_to_f64(to_host_raw(out, "bf16"), "bf16")
        rows = sample(c)
        ref = oat.prefill_chunk(codecs.decode(w.prompt_q[P0:P0 + C], "bf16"), P0, kc, vc,
                                pool.block_table(0), w.h_kv, w.sm_scale, "bf16", rows=rows)
        err = assert_close(got, ref, "bf16", f"mixed-prefill chunk {c}")
        say(f"    max|d| = {err:.3g}")
    kv.close()


def test_mixed_prefill_full_size_sampled():
    rng = np.random.default_rng(77)
    fixed = np.array([0, 1, 31, 32, 255, 256, 480, 510, 511])

    def sample(c):
        if c <= 1:
            return None  # every row
        return np.unique(np.concatenate([fixed, rng.choice(512, 7, replace=False)]))

    _mixed_prefix_run([0, 1, 31, 63], sample)


def test_slices_with_empty_slice_and_wide_groups_fp8():
    # a zero-length slice between two others; 16 query heads per KV head
    # (two head groups per work-group set), fp8 cache, head dim 64
    w = workloads.prefill_workload("empty-slice", 600, prompts=[500, 300],
                                   slices=[(0, 100, 77), (1, 50, 0), (1, 50, 130)],
                                   h_q=32, h_kv=2, d=64, cache_dtype="fp8")
    _check(w, "fp8 32/2 d64 with an empty slice")


def test_zero_work_calls_are_no_ops():
    import torch

    import paged_kv_cache_host_amd as pa
    from paged_kv_cache_host_amd.engine import PagedKV

    kv = PagedKV(8, 2, 64, "bf16", "cuda")
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    sl = torch.empty((0,), dtype=torch.int32, device="cuda")
    assert pa.pa_cache_write(None, e, e, sl, kv.k, kv.v, 8, 2, 64) == 0
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    lens = torch.zeros((0,), dtype=torch.int32, device="cuda")
    assert pa.pa_decode(None, out, q, kv.k, kv.v, tables, lens, 8, 2, 16,
                        0.125, 1.0, 1.0, None) == 0
    cu = torch.zeros((1,), dtype=torch.int32, device="cuda")
    st = torch.zeros((0,), dtype=torch.int32, device="cuda")
    assert pa.pa_prefill_chunk(None, out, q, cu, st, kv.k, kv.v, tables, 8, 2, 0, 16,
                               0.125, 1.0, 1.0, None) == 0
    torch.cuda.synchronize()
    kv.close()


@pytest.mark.parametrize("bs,cache_dt,d", [(8, "bf16", 128), (32, "bf16", 128), (8, "fp8", 128),
                                           (32, "fp8", 128), (8, "bf16", 64), (32, "fp8", 64)])
def test_block_sizes_8_and_32(bs, cache_dt, d):
    """pa_prefill_chunk over caches of 8- and 32-token blocks (ARTICLE 4.1):
    the C allocator's tables for that block size equal the oracle's; the cache
    is scattered here by layout alone (its bytes equal the oracle's scatter);
    outputs within tolerance of the oracle.  Prompts of 1, 9, 17 and 33
    tokens, slices starting off block boundaries, a 188-row tail and two
    slices of a 2500-token prompt (key ranges split over work-groups)."""
    import torch

    from oracle import allocator as oa
    from oracle import attention as oat
    from oracle import cache as oc
    from oracle import codecs
    import paged_kv_cache_host_amd._pa as pa
    from paged_kv_cache_host_amd.engine import prefill_workspace
    dev = "cuda"
    rng = np.random.default_rng(2300 + bs + d + len(cache_dt))
    prompts = [1, 9, 17, 33, 700, 2500]
    slices = [(0, 0, 1), (1, 0, 9), (2, 3, 14), (3, 16, 17), (4, 512, 188), (5, 1024, 512),
              (5, 1988, 512)]
    S, h_q, h_kv = len(prompts), 16, 2
    nb = sum(-(-P // bs) for P in prompts) + 5
    order = rng.permutation(nb).astype(np.int32)
    ntok = sum(prompts)
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
    T = sum(n for _, _, n in slices)
    q_raw = workloads.normal_raw(rng, (T, h_q, d), "bf16")
    # host side: the C allocator with this block size
    st_, pool = pa.pa_pool_create(nb, bs, order)
    assert st_ == pa.PA_OK
    try:
        slots = []
        for s, P in enumerate(prompts):
            assert pa.pa_seq_create(pool, s, P) == pa.PA_OK
            st_, sl = pa.pa_seq_slots(pool, s, 0, P)
            assert st_ == pa.PA_OK
            slots.append(np.asarray(sl, dtype=np.int64))
        mb = max(-(-P // bs) for P in prompts)
        st_, tables, _ = pa.pa_pack_batch(pool, np.array([s for s, _, _ in slices]), mb)
        assert st_ == pa.PA_OK
    finally:
        pa.pa_pool_destroy(pool)
    slots = np.concatenate(slots)
    opool = oa.BlockPool(nb, bs, order.tolist())
    for s, P in enumerate(prompts):
        assert opool.seq_create(s, P) == oa.OK
    o_slots = np.concatenate([np.asarray(opool.slots(s, 0, P)) for s, P in enumerate(prompts)])
    assert np.array_equal(o_slots, slots)
    for i, (s, _, _) in enumerate(slices):
        t = opool.block_table(s)
        assert list(tables[i, :len(t)]) == list(t)
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
    q64 = codecs.decode(q_raw, "bf16")
    cu = np.concatenate([[0], np.cumsum([n for _, _, n in slices])]).astype(np.int32)
    ref = np.concatenate([oat.prefill_chunk(q64[cu[i]:cu[i + 1]], a, okc, ovc,
                                            opool.block_table(s), h_kv, sm, cache_dt, ks, vs)
                          for i, (s, a, _) in enumerate(slices)])
    if cache_dt == "bf16":
        k_d = torch.from_numpy(kc.view(np.int16)).to(dev).view(torch.bfloat16)
        v_d = torch.from_numpy(vc.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        k_d = torch.from_numpy(kc).to(dev).view(torch.float8_e4m3fn)
        v_d = torch.from_numpy(vc).to(dev).view(torch.float8_e4m3fn)
    q_d = torch.from_numpy(q_raw.view(np.int16)).to(dev).view(torch.bfloat16)
    start = np.array([a for _, a, _ in slices], dtype=np.int32)
    max_q = max(n for _, _, n in slices)
    max_ctx = max(a + n for _, a, n in slices)
    out = filled((T, h_q, d), torch.bfloat16, dev)
    ws = prefill_workspace(len(slices), max_q, h_q, h_kv, d, max_ctx, dev)
    say(f"[prefill bs={bs}] {cache_dt} d={d} slices={slices} pool={nb}")
    assert pa.pa_prefill_chunk(None, out, q_d, torch.from_numpy(cu).to(dev),
                               torch.from_numpy(start).to(dev), k_d, v_d,
                               torch.from_numpy(tables).to(dev), nb, h_kv, max_q, max_ctx, sm,
                               ks, vs, ws, bs=bs) == 0
    torch.cuda.synchronize()
    got = codecs.decode(out.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    err = assert_close(got, ref, cache_dt, f"prefill bs={bs} {cache_dt} d={d}")
    say(f"    max|d| = {err:.3g}")
