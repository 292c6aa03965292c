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
    dev = torch.zeros(64, dtype=torch.int32, device=DEV)
    pageable = np.arange(64, dtype=np.int32)
    st = pa._lib.pa_stage(None, dev.data_ptr(), pageable.ctypes.data, 256)
    assert st == pa.PA_ERR_INVALID
    host = torch.arange(64, dtype=torch.int32).pin_memory()
    assert pa._lib.pa_stage(None, dev.data_ptr(), host.data_ptr() + 2, 8) == pa.PA_ERR_INVALID
    assert pa._lib.pa_stage(None, dev.data_ptr(), host.data_ptr(), 6) == pa.PA_ERR_INVALID
    assert pa._lib.pa_stage(None, dev.data_ptr(), host.data_ptr(), 0) == 0
    torch.cuda.synchronize()
    assert (dev.cpu() == 0).all()
    with pytest.raises(pa.PaError):
        pa.pa_stage(None, dev, torch.arange(64, dtype=torch.int32))
