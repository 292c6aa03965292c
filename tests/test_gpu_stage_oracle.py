"""GPU: the fused staging launches that the decode step and the trace run
(pa_stage_cache_write, pa_stage_decode_append, pa_decode_append), compared
directly with the oracle.

LESSON "The Concept: PagedAttention as a virtual memory system": token
position p of a sequence lives in physical block table[p // 16] at offset
p % 16, and a sequence's table grows by one block whenever its next token
crosses a block boundary (ARTICLE 2.2).  After every append the cache bytes
must equal oracle/cache.py's scatter of the same tokens into the same slots,
and every device block-table row must equal oracle/allocator.py's table of
that sequence over its context (entries past it untouched).  The slots come
from the library's host allocator, which the oracle's allocator must match
bit for bit as well; the device tables start as the oracle's tables."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_host_amd._pa as pa
import workloads
from oracle import allocator as oa
from oracle import cache as oc
from paged_kv_cache_host_amd.engine import _TORCH_STORAGE, to_device_raw, to_host_raw

pytestmark = pytest.mark.gpu

DEV = "cuda"
KS, VS = 0.03, 0.05     # fp8 per-tensor scales (ignored by the other caches)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _device_cache(nb, h_kv, d, cache_dt):
    dt = _TORCH_STORAGE[cache_dt]
    x = 16 // torch.empty((), dtype=dt).element_size()
    return (torch.zeros((nb, h_kv, d // x, 16, x), dtype=dt, device=DEV),
            torch.zeros((nb, h_kv, d, 16), dtype=dt, device=DEV))


def _assert_cache_equal(k_dev, v_dev, kc, vc, cache_dt, what):
    assert np.array_equal(to_host_raw(k_dev, cache_dt), kc), f"{what}: K cache bytes differ"
    assert np.array_equal(to_host_raw(v_dev, cache_dt), vc), f"{what}: V cache bytes differ"


@pytest.mark.parametrize("launch", ["stage_decode_append", "decode_append"])
@pytest.mark.parametrize("cache_dt,d", [("bf16", 128), ("fp8", 128), ("bf16", 64)])
def test_decode_append_against_oracle(launch, cache_dt, d):
    """A fixed decode batch grown by one token per iteration for 36
    iterations; contexts start at and beside block boundaries."""
    rng = np.random.default_rng(3100 + d + len(cache_dt) + len(launch))
    S, h_kv, steps = 29, 2, 36
    lengths = rng.integers(1, 60, size=S)
    lengths[:6] = [16, 32, 1, 15, 17, 48]
    MB = int(-(-(lengths.max() + steps) // 16))
    nb = int(sum(-(-(L + steps) // 16) for L in lengths)) + 6
    order = rng.permutation(nb).astype(np.int32)
    seqs = np.arange(S, dtype=np.int64)
    say(f"[decode append vs oracle] {launch} {cache_dt} d{d} S={S} steps={steps} pool={nb}")

    opool = oa.BlockPool(nb, 16, order.tolist())
    for s, L in enumerate(lengths):
        assert opool.seq_create(s, int(L)) == oa.OK
    kc, vc = oc.new_cache(nb, h_kv, 16, d, cache_dt)
    tables0, _ = opool.pack(range(S), MB)
    tables0 = np.asarray(tables0, dtype=np.int32)
    d_tab = torch.from_numpy(tables0.copy()).to(DEV)
    k_dev, v_dev = _device_cache(nb, h_kv, d, cache_dt)

    st, pool = pa.pa_pool_create(nb, 16, order)
    assert st == pa.PA_OK
    try:
        for s, L in enumerate(lengths):
            assert pa.pa_seq_create(pool, s, int(L)) == pa.PA_OK
        lens = lengths.astype(np.int32).copy()
        host = torch.empty(2 * S, dtype=torch.int32, pin_memory=True)
        h = host.numpy()
        staged = torch.empty(2 * S, dtype=torch.int32, device=DEV)
        for it in range(steps):
            st, done, slots = pa.pa_batch_append(pool, seqs, 1)
            assert st == pa.PA_OK and done == S
            o_slots = []
            for s in range(S):
                ost, sl = opool.seq_append(s, 1)
                assert ost == oa.OK
                o_slots += sl
            assert slots[:, 0].tolist() == o_slots, it
            lens += 1
            k_raw = workloads.normal_raw(rng, (S, h_kv, d), "bf16")
            v_raw = workloads.normal_raw(rng, (S, h_kv, d), "bf16")
            kn = to_device_raw(k_raw, "bf16", DEV)
            vn = to_device_raw(v_raw, "bf16", DEV)
            h[:S] = slots[:, 0]
            h[S:] = lens
            if launch == "stage_decode_append":
                assert pa.pa_stage_decode_append(None, staged, host, 8 * S, 0, 4 * S, S, kn, vn,
                                                 k_dev, v_dev, nb, h_kv, d, d_tab, 16, KS,
                                                 VS) == pa.PA_OK
            else:
                assert pa.pa_stage(None, staged, host, 8 * S) == pa.PA_OK
                assert pa.pa_decode_append(None, staged[:S], staged[S:], S, kn, vn, k_dev, v_dev,
                                           nb, h_kv, d, d_tab, 16, KS, VS) == pa.PA_OK
            torch.cuda.synchronize()
            oc.cache_write(kc, vc, k_raw, v_raw, o_slots, "bf16", cache_dt, KS, VS)
            got = d_tab.cpu().numpy()
            for s in range(S):
                t = opool.block_table(s)
                assert got[s, :len(t)].tolist() == t, (it, s)
                assert (got[s, len(t):] == -1).all(), (it, s)
            assert np.array_equal(staged.cpu().numpy(), h), it
            if it % 6 == 0 or it == steps - 1:
                _assert_cache_equal(k_dev, v_dev, kc, vc, cache_dt, f"iteration {it}")
    finally:
        pa.pa_pool_destroy(pool)


@pytest.mark.parametrize("new_dt,cache_dt,d", [("bf16", "bf16", 128), ("bf16", "fp8", 128),
                                               ("bf16", "bf16", 64), ("f32", "f32", 64)])
def test_stage_cache_write_against_oracle(new_dt, cache_dt, d):
    """Scheduler-style iterations: prefill slices and decode tokens of
    several sequences (slots from the oracle's allocator, a few skipped with
    -1), staged with padding words around the slots; the device copy must
    equal the host buffer and the cache bytes the oracle's scatter after
    every launch."""
    rng = np.random.default_rng(3200 + d + len(cache_dt))
    h_kv, nb = 4, 96
    prompts = [130, 17, 1, 64, 250]
    order = rng.permutation(nb).astype(np.int32)
    say(f"[stage cache write vs oracle] {new_dt}->{cache_dt} d{d} pool={nb}")
    opool = oa.BlockPool(nb, 16, order.tolist())
    for s, P in enumerate(prompts):
        assert opool.seq_create(s, P) == oa.OK
    kc, vc = oc.new_cache(nb, h_kv, 16, d, cache_dt)
    k_dev, v_dev = _device_cache(nb, h_kv, d, cache_dt)
    # iterations: (sequence, first position, count) pieces written together
    iterations = [[(0, 0, 64), (1, 0, 17)], [(0, 64, 66), (2, 0, 1), (3, 0, 33)],
                  [(3, 33, 31), (4, 0, 200)], [(4, 200, 50)]]
    for it, pieces in enumerate(iterations):
        slots = np.concatenate([opool.slots(s, a, n) for s, a, n in pieces]).astype(np.int32)
        n = len(slots)
        if n >= 4:
            slots[[1, n - 2]] = -1          # skipped tokens
        pad = 3 + it
        words = pad + n + 5
        host = torch.empty(words, dtype=torch.int32, pin_memory=True)
        hv = host.numpy()
        hv[:] = rng.integers(-2**31, 2**31 - 1, size=words, dtype=np.int64).astype(np.int32)
        hv[pad:pad + n] = slots
        k_raw = workloads.normal_raw(rng, (n, h_kv, d), new_dt)
        v_raw = workloads.normal_raw(rng, (n, h_kv, d), new_dt)
        kn = to_device_raw(k_raw, new_dt, DEV)
        vn = to_device_raw(v_raw, new_dt, DEV)
        dst = torch.full((words,), -9, dtype=torch.int32, device=DEV)
        assert pa.pa_stage_cache_write(None, dst, host, 4 * words, 4 * pad, n, kn, vn, k_dev,
                                       v_dev, nb, h_kv, d, 16, KS, VS) == pa.PA_OK
        torch.cuda.synchronize()
        oc.cache_write(kc, vc, k_raw, v_raw, slots, new_dt, cache_dt, KS, VS)
        assert np.array_equal(dst.cpu().numpy(), hv), it
        _assert_cache_equal(k_dev, v_dev, kc, vc, cache_dt, f"iteration {it}")
