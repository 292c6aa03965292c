"""GPU: pa_stage moves pinned host bytes into device memory exactly, through
the C ABI — sizes that do and do not fill whole work-groups, sources inside
an allocation, the same pinned buffer rewritten between calls (host writes
must be seen, never stale data) — and rejects sources that are not pinned
or not aligned without launching anything."""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_host_amd._pa as pa

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_stage_sizes_and_offsets():
    rng = np.random.default_rng(900)
    host = torch.empty(1 << 20, dtype=torch.int32, pin_memory=True)
    dev = torch.empty(1 << 20, dtype=torch.int32, device=DEV)
    # words: 1, one thread short of / exactly / one past a work-group's
    # 256 x 4 words, many work-groups, more than the 256-group grid covers
    for words, off in [(1, 0), (1023, 0), (1024, 0), (1025, 3), (30000, 17), (300000, 5),
                       ((1 << 20) - 9, 9)]:
        say(f"[stage] words={words} offset={off}")
        h = host.numpy()
        h[:] = rng.integers(-2**31, 2**31 - 1, size=h.size, dtype=np.int64).astype(np.int32)
        dev.fill_(-7)
        assert pa.pa_stage(None, dev[off:off + words], host[off:off + words]) == 0
        torch.cuda.synchronize()
        got = dev.cpu().numpy()
        assert np.array_equal(got[off:off + words], h[off:off + words])
        assert (got[:off] == -7).all() and (got[off + words:] == -7).all()


def test_stage_sees_every_host_rewrite():
    """Two pinned buffers by parity, each rewritten by the host before every
    other call, as the per-iteration metadata is; every call's device copy
    must hold that call's bytes."""
    rng = np.random.default_rng(901)
    n = 30000
    host = [torch.empty(n, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    dev = torch.empty((24, n), dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    done = [torch.cuda.Event() for _ in range(2)]
    want = []
    for i in range(24):
        X = i & 1
        done[X].synchronize()
        v = rng.integers(0, 1 << 30, size=n, dtype=np.int64).astype(np.int32)
        host[X].numpy()[:] = v
        want.append(v)
        assert pa.pa_stage(s, dev[i], host[X]) == 0
        done[X].record(s)
    s.synchronize()
    got = dev.cpu().numpy()
    for i in range(24):
        assert np.array_equal(got[i], want[i]), i


def test_stage_rejects_bad_sources():
    """Pageable sources are refused by the host-only check every staging
    launch makes first (pa_pinned_alias, which never launches); misaligned
    pinned sources and sizes reach pa_stage itself, with real buffers on
    both sides, so nothing outside them can be touched."""
    dev = torch.zeros(64, dtype=torch.int32, device=DEV)
    pageable = np.arange(64, dtype=np.int32)
    st, alias = pa.pa_pinned_alias(pageable.ctypes.data)
    assert st == pa.PA_ERR_INVALID and alias == 0
    host = torch.arange(64, dtype=torch.int32).pin_memory()
    st, alias = pa.pa_pinned_alias(host.data_ptr())
    assert st == pa.PA_OK and alias != 0
    assert pa._lib.pa_stage(None, dev.data_ptr(), host.data_ptr() + 2, 8) == pa.PA_ERR_INVALID
    assert pa._lib.pa_stage(None, dev.data_ptr(), host.data_ptr(), 6) == pa.PA_ERR_INVALID
    assert pa._lib.pa_stage(None, dev.data_ptr(), host.data_ptr(), 0) == 0
    torch.cuda.synchronize()
    assert (dev.cpu() == 0).all()
    with pytest.raises(pa.PaError):
        pa.pa_stage(None, dev, torch.arange(64, dtype=torch.int32))


@pytest.mark.parametrize("new_dt,cache_dt,d", [("bf16", "bf16", 128), ("bf16", "fp8", 128),
                                               ("bf16", "bf16", 64), ("f32", "f32", 64)])
def test_stage_cache_write_equals_stage_then_cache_write(new_dt, cache_dt, d):
    """The fused launch leaves the same device copy and the same cache bytes
    as pa_stage followed by pa_cache_write: several sizes (whole and partial
    work-groups of tokens, 4- and 8-byte words), slots that are skipped (-1)
    or lie outside the pool, on the same buffers twice in a row."""
    from paged_kv_cache_host_amd.engine import _TORCH_STORAGE
    rng = np.random.default_rng(902)
    h_kv, nb = 4, 40
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[new_dt]
    cdt = _TORCH_STORAGE[cache_dt]
    x = 16 // torch.empty((), dtype=cdt).element_size()
    caches = []
    for _ in range(2):
        k = torch.zeros((nb, h_kv, d // x, 16, x), dtype=cdt, device=DEV)
        v = torch.zeros((nb, h_kv, d, 16), dtype=cdt, device=DEV)
        caches.append((k, v))
    g = torch.Generator(device=DEV)
    g.manual_seed(903)
    for n, pad_words in [(0, 10), (1, 3), (17, 0), (200, 501), (33, 2)]:
        say(f"[stage_cache_write] {new_dt}->{cache_dt} d{d} n={n} pad={pad_words}")
        words = pad_words + n + 5
        slot_off = 4 * pad_words
        host = torch.empty(words, dtype=torch.int32, pin_memory=True)
        h = host.numpy()
        h[:] = rng.integers(-2**31, 2**31 - 1, size=words, dtype=np.int64).astype(np.int32)
        sl = rng.permutation(nb * 16)[:n].astype(np.int32)
        if n >= 3:
            sl[1] = -1
            sl[2] = nb * 16 + 7        # outside the pool: skipped
        h[pad_words:pad_words + n] = sl
        kn = torch.randn((max(n, 1), h_kv, d), generator=g, device=DEV).to(tdt)
        vn = torch.randn((max(n, 1), h_kv, d), generator=g, device=DEV).to(tdt)
        outs = []
        for i, (kc, vc) in enumerate(caches):
            dst = torch.full((words + 3,), -9, dtype=torch.int32, device=DEV)
            if i == 0:
                assert pa.pa_stage(None, dst, host, 4 * words) == 0
                if n:
                    assert pa.pa_cache_write(None, kn, vn, dst[pad_words:pad_words + n], kc, vc,
                                             nb, h_kv, d, 16, 0.03, 0.05) == 0
            else:
                assert pa.pa_stage_cache_write(None, dst, host, 4 * words, slot_off, n, kn, vn,
                                               kc, vc, nb, h_kv, d, 16, 0.03, 0.05) == 0
            torch.cuda.synchronize()
            outs.append(dst.cpu())
        assert torch.equal(outs[0], outs[1])
        for a, b in zip(caches[0], caches[1]):
            assert torch.equal(a.view(torch.uint8).cpu(), b.view(torch.uint8).cpu())


def test_stage_cache_write_rejects_bad_arguments():
    """Every device argument is a real buffer sized for the call (10 blocks
    of 2 KV heads x 64 dims, 8 new tokens whose slots, read from the pinned
    buffer, lie inside the pool), so that even a launch after a failed check
    would stay inside them; the pageable source goes to the host-only check."""
    host = torch.arange(64, dtype=torch.int32).pin_memory()
    lib = pa._lib
    nb, h_kv, d, n = 10, 2, 64, 8
    dst = torch.zeros(64 + 16, dtype=torch.int32, device=DEV)
    kn = torch.zeros((n, h_kv, d), dtype=torch.bfloat16, device=DEV)
    vn = torch.zeros((n, h_kv, d), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((nb, h_kv, d // 8, 16, 8), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((nb, h_kv, d, 16), dtype=torch.bfloat16, device=DEV)
    args = (kn.data_ptr(), vn.data_ptr(), 1)
    cache = (kc.data_ptr(), vc.data_ptr(), 1, nb, h_kv, d, 16, 1.0, 1.0)
    # 8 slots at byte 40 of a 64-byte buffer, then a misaligned slot offset
    assert lib.pa_stage_cache_write(None, dst.data_ptr(), host.data_ptr(), 64, 40, *args, n,
                                    *cache) == pa.PA_ERR_INVALID
    assert lib.pa_stage_cache_write(None, dst.data_ptr(), host.data_ptr(), 64, 2, *args, 1,
                                    *cache) == pa.PA_ERR_INVALID
    torch.cuda.synchronize()
    assert (dst.cpu() == 0).all() and (kc.view(torch.int16).cpu() == 0).all()
    pageable = np.zeros(64, dtype=np.int32)
    assert pa.pa_pinned_alias(pageable.ctypes.data)[0] == pa.PA_ERR_INVALID


@pytest.mark.parametrize("device_meta", [False, True], ids=["staged", "device"])
@pytest.mark.parametrize("cache_dt,d", [("bf16", 128), ("fp8", 128), ("bf16", 64)])
def test_stage_decode_append_keeps_device_tables(cache_dt, d, device_meta):
    """Decode iterations whose block tables stay on the device: after every
    iteration each row equals the allocator's table (pa_pack_batch) entry for
    entry over its context, and the cache bytes and the staged copy equal
    those of pa_stage_cache_write on the same data.  Contexts start at and
    around block boundaries; one iteration carries a slot outside the pool
    and a length beyond the row, which leave their rows unchanged.
    ``device``: pa_decode_append reads the slots and lengths that
    pa_stage_cache_write staged into device memory."""
    from paged_kv_cache_host_amd.engine import _TORCH_STORAGE
    rng = np.random.default_rng(911)
    S, h_kv, steps = 37, 2, 40
    lengths = rng.integers(1, 70, size=S)
    lengths[:5] = [16, 32, 1, 15, 17]
    MB = int(-(-(lengths.max() + steps) // 16))
    nb = int(sum(-(-(L + steps) // 16) for L in lengths)) + 8
    st_, pool = pa.pa_pool_create(nb, 16, rng.permutation(nb).astype(np.int32))
    assert st_ == pa.PA_OK
    seqs = np.arange(S, dtype=np.int64)
    try:
        for s, L in enumerate(lengths):
            assert pa.pa_seq_create(pool, s, int(L) - 1) == pa.PA_OK
        st_, tab0, lens = pa.pa_pack_batch(pool, seqs, MB)
        assert st_ == pa.PA_OK
        d_tab = torch.from_numpy(tab0.copy()).to(DEV)
        cdt = _TORCH_STORAGE[cache_dt]
        x = 16 // torch.empty((), dtype=cdt).element_size()
        caches = [(torch.zeros((nb, h_kv, d // x, 16, x), dtype=cdt, device=DEV),
                   torch.zeros((nb, h_kv, d, 16), dtype=cdt, device=DEV)) for _ in range(2)]
        host = torch.empty(2 * S + 3, dtype=torch.int32, pin_memory=True)
        h = host.numpy()
        g = torch.Generator(device=DEV)
        g.manual_seed(912)
        say(f"[stage_decode_append] {cache_dt} d{d} S={S} steps={steps} max_blocks={MB} "
            f"device_meta={device_meta}")
        for it in range(steps):
            st_, done, slots = pa.pa_batch_append(pool, seqs, 1)
            assert st_ == pa.PA_OK and done == S
            lens = lens + 1
            h[:S] = slots[:, 0]
            h[S:2 * S] = lens
            h[2 * S:] = it
            edge = it == steps // 2
            if edge:
                h[5] = nb * 16 + 3        # slot outside the pool: row 5 unchanged
                h[S + 6] = MB * 16 + 1    # length beyond the row: row 6 unchanged
            before = d_tab.cpu()
            kn = torch.randn((S, h_kv, d), generator=g, device=DEV).to(torch.bfloat16)
            vn = torch.randn((S, h_kv, d), generator=g, device=DEV).to(torch.bfloat16)
            dsts = [torch.full((2 * S + 5,), -7, dtype=torch.int32, device=DEV) for _ in range(2)]
            assert pa.pa_stage_cache_write(None, dsts[0], host, 4 * (2 * S + 3), 0, S, kn, vn,
                                           caches[0][0], caches[0][1], nb, h_kv, d, 16, 0.03,
                                           0.05) == 0
            if device_meta:
                assert pa.pa_decode_append(None, dsts[0][:S], dsts[0][S:2 * S], S, kn, vn,
                                           caches[1][0], caches[1][1], nb, h_kv, d, d_tab, 16,
                                           0.03, 0.05) == 0
            else:
                assert pa.pa_stage_decode_append(None, dsts[1], host, 4 * (2 * S + 3), 0, 4 * S,
                                                 S, kn, vn, caches[1][0], caches[1][1], nb, h_kv,
                                                 d, d_tab, 16, 0.03, 0.05) == 0
            torch.cuda.synchronize()
            if not device_meta:
                assert torch.equal(dsts[0].cpu(), dsts[1].cpu())
            for a, b in zip(caches[0], caches[1]):
                assert torch.equal(a.view(torch.uint8).cpu(), b.view(torch.uint8).cpu())
            got = d_tab.cpu().numpy()
            st_, ref, _ = pa.pa_pack_batch(pool, seqs, MB)
            assert st_ == pa.PA_OK
            for i in range(S):
                nblk = -(-int(lens[i]) // 16)
                if edge and i in (5, 6):
                    assert np.array_equal(got[i], before[i].numpy()), (it, i)
                    got[i, :nblk] = ref[i, :nblk]      # the host repairs the row
                    d_tab[i] = torch.from_numpy(ref[i].copy()).to(DEV)
                assert np.array_equal(got[i, :nblk], ref[i, :nblk]), (it, i)
                # entries past the context are never written
                assert np.array_equal(got[i, nblk:], tab0[i, nblk:]), (it, i)
    finally:
        pa.pa_pool_destroy(pool)
