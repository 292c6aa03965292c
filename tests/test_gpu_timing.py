"""GPU: the kernel-timing facility (pa_timing_*) times exactly the selected
kernels' launches, and their durations fit inside the stream's elapsed
time around them."""
import numpy as np
import pytest
import torch

import paged_kv_cache_host_amd._pa as pa
from paged_kv_cache_host_amd.engine import PagedKV, decode_workspace

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_timing_keeps_selected_kernels_and_adds_up():
    lengths = [300, 2000, 4100, 17]
    nb = sum(-(-L // 16) for L in lengths) + 3
    kv = PagedKV(nb, 8, 128, "bf16", DEV, None)
    g = torch.Generator(device=DEV)
    g.manual_seed(12)
    slots = []
    for s, L in enumerate(lengths):
        pa.check(kv.create(s, L))
        slots.append(kv.slots(s, 0, L))
    slots = torch.from_numpy(np.concatenate(slots).astype(np.int32)).to(DEV)
    n = slots.numel()
    k = torch.randn((n, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((n, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    tables, lens = kv.pack(list(range(len(lengths))))
    t_d, l_d = torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV)
    q = torch.randn((len(lengths), 64, 128), generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty_like(q)
    ws = decode_workspace(len(lengths), 64, 8, 128, max(lengths), DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pa.check(pa.pa_timing_enable(["decode"]))
    a.record(s)
    kv.write(k, v, slots, stream=s)
    for _ in range(10):
        kv.decode(out, q, t_d, l_d, max(lengths), 1 / 128 ** 0.5, ws, stream=s)
    b.record(s)
    s.synchronize()
    st, cnt, mean_us, tot_us = pa.pa_timing_query("decode")
    pa.check(st)
    assert cnt == 10
    st, cnt_cw, _, _ = pa.pa_timing_query("cache_write")
    pa.check(st)
    assert cnt_cw == 0                               # not selected
    wall_us = a.elapsed_time(b) * 1e3
    assert 0 < tot_us <= wall_us, (tot_us, wall_us)
    pa.check(pa.pa_timing_enable(True, every=3))
    for _ in range(10):
        kv.decode(out, q, t_d, l_d, max(lengths), 1 / 128 ** 0.5, ws, stream=s)
    s.synchronize()
    assert pa.pa_timing_query("decode")[1] == 4        # launches 0, 3, 6, 9; earlier ones forgotten
    pa.check(pa.pa_timing_enable(False))
    kv.close()
