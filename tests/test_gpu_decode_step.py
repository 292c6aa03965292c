"""GPU: pa_decode_step -- the new tokens' K/V into their slots, the block
tables' new entries and decode attention, in one launch -- against the
oracle, and bit for bit against the separate launches it replaces
(pa_stage_decode_append + pa_decode).

LESSON "Continuous batching at the iteration level": every iteration writes
the new tokens' K/V before attention reads the cache, so the decode at
position L-1 sees context length L (its own token included).  ARTICLE 2.2:
a sequence's block table gains an entry when its next token opens a block.
After every iteration the output must pass the parity gate against
oracle/attention.py's decode over oracle/cache.py's scatter of the same
tokens, the device tables must equal oracle/allocator.py's tables and the
cache bytes the oracle's."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_host_amd as pa
from oracle import allocator as oa
from oracle import attention as oat
from oracle import cache as oc
from oracle import codecs
from paged_kv_cache_host_amd.engine import decode_workspace, to_device_raw, to_host_raw
from tests.gate import SENTINEL, assert_close
from tests.parity import out_to_f64
from tests.step_parity import KS, VS, StepBatch, _blocks, _meta

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _step(b, dst, host, nbytes, slot_off, lens_off, kn, vn, out, q, ws, max_ctx, device_meta):
    if device_meta:
        assert pa.pa_stage(None, dst, host, nbytes) == pa.PA_OK
        src = None
    else:
        src = host
    return pa.pa_decode_step(None, dst, src, nbytes, slot_off, lens_off, kn, vn, out, q, b.k_dev,
                             b.v_dev, b.tab_dev, b.nb, b.h_kv, max_ctx, b.sm, KS, VS, ws)


CASES = {
    "bf16-d128": ("bf16", 128),
    "fp8-d128": ("fp8", 128),
    "bf16-d64": ("bf16", 64),
    "fp8-d64": ("fp8", 64),
}


@pytest.mark.parametrize("device_meta", [False, True], ids=["staged", "device"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_step_against_oracle(case, device_meta):
    """Contexts from empty (the first token opens block 0) through block
    edges to several 2048-token chunks (merged by the second kernel); five
    iterations move contexts across block edges."""
    cache_dt, d = CASES[case]
    lengths = [0, 1, 14, 15, 16, 17, 31, 32, 47, 100, 2046, 2047, 2048, 4100, 700, 5, 63, 64,
               333, 1000, 18, 9, 2500]
    steps = 5
    b = StepBatch(5100 + d + len(cache_dt) + device_meta, lengths, 16, 2, d, cache_dt, steps)
    say(f"[decode step vs oracle] {case} {'device' if device_meta else 'staged'} S={b.S} "
        f"pool={b.nb} max_blocks={b.mb}")
    ws = decode_workspace(b.S, b.h_q, b.h_kv, d, int(b.lengths.max()) + steps, DEV)
    for it in range(steps):
        slots, k, v, q = b.next_tokens()
        host, slot_off, lens_off, nbytes = _meta(b.S, slots, b.lens, pad=3 + it)
        dst = torch.full((nbytes // 4 + 2,), -7, dtype=torch.int32, device=DEV)
        out = torch.full((b.S, b.h_q, d), SENTINEL, dtype=torch.bfloat16, device=DEV)
        kn = to_device_raw(k, "bf16", DEV)
        vn = to_device_raw(v, "bf16", DEV)
        qd = to_device_raw(q, "bf16", DEV)
        max_ctx = int(b.lens.max())
        assert _step(b, dst, host, nbytes, slot_off, lens_off, kn, vn, out, qd, ws, max_ctx,
                     device_meta) == pa.PA_OK
        torch.cuda.synchronize()
        ref, tables = b.oracle_step(slots, k, v, q)
        err = assert_close(out_to_f64(to_host_raw(out, "bf16"), "bf16"), ref, cache_dt,
                           f"{case} iteration {it}")
        got_t = b.tab_dev.cpu().numpy()
        for s in range(b.S):
            n = _blocks(b.lens[s])
            assert np.array_equal(got_t[s, :n], tables[s, :n]), (it, s)
            assert (got_t[s, n:] == -1).all(), (it, s)
        got_dst = dst.cpu().numpy()
        assert np.array_equal(got_dst[:nbytes // 4], host.numpy()), it
        assert (got_dst[nbytes // 4:] == -7).all(), it
        assert int(ws[:64].view(torch.int32)[:3].abs().sum()) == 0, "counters left nonzero"
        if it in (0, steps - 1):
            assert np.array_equal(to_host_raw(b.k_dev, cache_dt), b.kc), f"K cache, iteration {it}"
            assert np.array_equal(to_host_raw(b.v_dev, cache_dt), b.vc), f"V cache, iteration {it}"
        say(f"  iteration {it}: max|d| = {err:.3g}")


def _two_launch_step(b, tab, k_dev, v_dev, dst, host, nbytes, slot_off, lens_off, kn, vn, out, q,
                     ws, max_ctx):
    assert pa.pa_stage_decode_append(None, dst, host, nbytes, slot_off, lens_off, b.S, kn, vn,
                                     k_dev, v_dev, b.nb, b.h_kv, b.d, tab, 16, KS,
                                     VS) == pa.PA_OK
    lens_dev = dst[lens_off // 4:lens_off // 4 + b.S]
    assert pa.pa_decode(None, out, q, k_dev, v_dev, tab, lens_dev, b.nb, b.h_kv, max_ctx, b.sm,
                        KS, VS, ws) == pa.PA_OK


@pytest.mark.parametrize("cache_dt", ["bf16", "fp8"])
def test_decode_step_equals_two_launches(cache_dt):
    """The 70B-shaped batch (128 sequences, 64/8 heads, d 128, lognormal
    contexts of mean ~1500 plus one of 9000 tokens, cut into two 8192-token
    chunks): outputs, cache bytes, tables and the staged copy equal those of
    pa_stage_decode_append + pa_decode over four iterations."""
    rng = np.random.default_rng(5200 + len(cache_dt))
    S, h_q, h_kv, d, steps = 128, 64, 8, 128, 4
    lengths = np.clip(np.round(rng.lognormal(np.log(1500) - 0.18, 0.6, size=S)), 1, 6000)
    lengths[7] = 9000
    lengths[8], lengths[9], lengths[10] = 15, 16, 31
    lengths = lengths.astype(np.int64)
    mb = _blocks(lengths.max() + steps)
    nb = int(sum(_blocks(L + steps) for L in lengths)) + 8
    pool = oa.BlockPool(nb, 16, rng.permutation(nb).astype(np.int32).tolist())
    for s, L in enumerate(lengths.tolist()):
        assert pool.seq_create(s, int(L)) == oa.OK
    tables, _ = pool.pack(range(S), mb)
    tab = [torch.from_numpy(np.asarray(tables, dtype=np.int32)).to(DEV) for _ in range(2)]
    g = torch.Generator(device=DEV)
    g.manual_seed(5201)
    x = 8 if cache_dt == "bf16" else 16
    if cache_dt == "bf16":
        k0 = torch.randn((nb, h_kv, d // x, 16, x), generator=g, device=DEV).to(torch.bfloat16)
        v0 = torch.randn((nb, h_kv, d, 16), generator=g, device=DEV).to(torch.bfloat16)
    else:
        # any byte but the two NaN codes (0x7f, 0xff)
        k0 = torch.randint(0, 127, (nb, h_kv, d // x, 16, x), generator=g, device=DEV,
                           dtype=torch.int32)
        k0 = (k0 + 128 * torch.randint(0, 2, k0.shape, generator=g, device=DEV,
                                       dtype=torch.int32)).to(torch.uint8)
        v0 = torch.randint(0, 127, (nb, h_kv, d, 16), generator=g, device=DEV,
                           dtype=torch.int32)
        v0 = (v0 + 128 * torch.randint(0, 2, v0.shape, generator=g, device=DEV,
                                       dtype=torch.int32)).to(torch.uint8)
    caches = [(k0.clone(), v0.clone()), (k0, v0)]

    class B:
        pass
    b = B()
    b.S, b.h_kv, b.d, b.nb, b.sm = S, h_kv, d, nb, 1.0 / np.sqrt(d)
    lens = lengths.astype(np.int32).copy()
    max_ctx = int(lengths.max()) + steps
    ws = [decode_workspace(S, h_q, h_kv, d, max_ctx, DEV) for _ in range(2)]
    say(f"[decode step vs two launches] {cache_dt} S={S} pool={nb} max_blocks={mb}")
    for it in range(steps):
        slots = []
        for s in range(S):
            st, sl = pool.seq_append(s, 1)
            assert st == oa.OK
            slots += sl
        lens += 1
        host, slot_off, lens_off, nbytes = _meta(S, np.asarray(slots, dtype=np.int32), lens,
                                                 pad=1 + it)
        kn = torch.randn((S, h_kv, d), generator=g, device=DEV).to(torch.bfloat16)
        vn = torch.randn((S, h_kv, d), generator=g, device=DEV).to(torch.bfloat16)
        q = torch.randn((S, h_q, d), generator=g, device=DEV).to(torch.bfloat16)
        dsts = [torch.full((nbytes // 4,), -7, dtype=torch.int32, device=DEV) for _ in range(2)]
        outs = [torch.full((S, h_q, d), SENTINEL, dtype=torch.bfloat16, device=DEV)
                for _ in range(2)]
        _two_launch_step(b, tab[0], caches[0][0], caches[0][1], dsts[0], host, nbytes, slot_off,
                         lens_off, kn, vn, outs[0], q, ws[0], max_ctx)
        assert pa.pa_decode_step(None, dsts[1], host, nbytes, slot_off, lens_off, kn, vn,
                                 outs[1], q, caches[1][0], caches[1][1], tab[1], nb, h_kv,
                                 max_ctx, b.sm, KS, VS, ws[1]) == pa.PA_OK
        torch.cuda.synchronize()
        a, c = (to_host_raw(o, "bf16") for o in outs)
        diff = np.flatnonzero(a.reshape(-1) != c.reshape(-1))
        assert diff.size == 0, f"iteration {it}: {diff.size} outputs differ"
        assert not (a == np.uint16(0x4640)).any(), "rows left unwritten"   # bf16 12288
        assert torch.equal(tab[0], tab[1]), it
        assert torch.equal(dsts[0], dsts[1]), it
        for u, w in zip(caches[0], caches[1]):
            assert torch.equal(u.view(torch.uint8), w.view(torch.uint8)), it
        say(f"  iteration {it}: identical")


def test_decode_step_edge_tokens():
    """A slot outside the pool (on a token that opens a block) and a length
    beyond the row leave their rows unchanged and write no K/V; every other
    row is written and attended as the oracle's."""
    b = StepBatch(5300, [20, 40, 16, 15, 2100, 3, 70], 16, 2, 128, "bf16", steps=1)
    ws = decode_workspace(b.S, b.h_q, b.h_kv, 128, 4096, DEV)
    slots, k, v, q = b.next_tokens()
    lens = b.lens.copy()
    bad_slot = slots.copy()
    bad_slot[2] = b.nb * 16 + 5          # row 2: slot outside the pool
    lens[5] = b.mb * 16 + 1              # row 5: length beyond the row
    host, slot_off, lens_off, nbytes = _meta(b.S, bad_slot, lens, pad=0)
    dst = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    out = torch.full((b.S, b.h_q, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    before_t = b.tab_dev.cpu().numpy().copy()
    say("[decode step] slot outside the pool, length beyond the row")
    assert pa.pa_decode_step(None, dst, host, nbytes, slot_off, lens_off,
                             to_device_raw(k, "bf16", DEV), to_device_raw(v, "bf16", DEV), out,
                             to_device_raw(q, "bf16", DEV), b.k_dev, b.v_dev, b.tab_dev, b.nb,
                             b.h_kv, 4096, b.sm, KS, VS, ws) == pa.PA_OK
    torch.cuda.synchronize()
    got_t = b.tab_dev.cpu().numpy()
    assert np.array_equal(got_t[2], before_t[2]) and np.array_equal(got_t[5], before_t[5])
    keep = np.ones(b.S, dtype=bool)
    keep[[2, 5]] = False
    oc.cache_write(b.kc, b.vc, k[keep], v[keep], slots[keep], "bf16", "bf16")
    assert np.array_equal(to_host_raw(b.k_dev, "bf16"), b.kc)
    assert np.array_equal(to_host_raw(b.v_dev, "bf16"), b.vc)
    tables, _ = b.pool.pack(range(b.S), b.mb)
    tables = np.asarray(tables, dtype=np.int32)
    rows = np.flatnonzero(keep)
    for s in rows:
        n = _blocks(b.lens[s])
        assert np.array_equal(got_t[s, :n], tables[s, :n]), s
    ref = oat.decode(codecs.decode(q, "bf16")[rows], b.kc, b.vc, tables[rows], b.lens[rows],
                     b.h_kv, b.sm, "bf16")
    got = out_to_f64(to_host_raw(out, "bf16"), "bf16")
    assert np.isfinite(got).all()
    assert_close(got[rows], ref, "bf16", "edge tokens: the other rows")
    assert int(ws[:64].view(torch.int32)[:3].abs().sum()) == 0


def test_decode_step_workspace_serves_smaller_calls():
    """One workspace sized for the largest batch serves, in turn, batches
    with fewer sequences and shorter contexts (fewer chunks), each checked
    against the oracle and each leaving the work counters zero."""
    specs = [([3000, 70, 5000, 16, 1, 900, 2047, 33], 2),
             ([10, 31], 2),
             ([4097, 12, 600], 2)]
    batches = [StepBatch(5400 + i, L, 16, 2, 128, "bf16", steps=st)
               for i, (L, st) in enumerate(specs)]
    ws = decode_workspace(8, 16, 2, 128, 8192, DEV)
    for rep in range(2):
        for i, b in enumerate(batches):
            slots, k, v, q = b.next_tokens()
            host, slot_off, lens_off, nbytes = _meta(b.S, slots, b.lens, pad=i)
            dst = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
            out = torch.full((b.S, b.h_q, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
            say(f"[decode step shared workspace] batch {i} rep {rep}: S={b.S}")
            assert pa.pa_decode_step(None, dst, host, nbytes, slot_off, lens_off,
                                     to_device_raw(k, "bf16", DEV),
                                     to_device_raw(v, "bf16", DEV), out,
                                     to_device_raw(q, "bf16", DEV), b.k_dev, b.v_dev, b.tab_dev,
                                     b.nb, b.h_kv, int(b.lens.max()), b.sm, KS, VS,
                                     ws) == pa.PA_OK
            torch.cuda.synchronize()
            ref, _ = b.oracle_step(slots, k, v, q)
            assert_close(out_to_f64(to_host_raw(out, "bf16"), "bf16"), ref, "bf16",
                         f"batch {i} rep {rep}")
            assert int(ws[:64].view(torch.int32)[:3].abs().sum()) == 0


def test_decode_step_bounded_wait_path():
    """With the poll limit lowered to one poll, the work-groups that do not
    see the staged metadata at once take no work and end; work-group 0 (and
    any that did see it) serve the whole queue.  Results as the oracle's
    over three iterations, with a context long enough to span chunks."""
    b = StepBatch(5500, [3, 700, 2049, 16, 15, 90, 4097, 1], 16, 2, 128, "bf16", steps=3)
    ws = decode_workspace(b.S, b.h_q, b.h_kv, 128, int(b.lengths.max()) + 3, DEV)
    assert pa.pa_decode_step_set_spin_limit(1) == pa.PA_OK
    try:
        for it in range(3):
            slots, k, v, q = b.next_tokens()
            host, slot_off, lens_off, nbytes = _meta(b.S, slots, b.lens, pad=it)
            dst = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
            out = torch.full((b.S, b.h_q, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
            say(f"[decode step, one poll] iteration {it}")
            assert pa.pa_decode_step(None, dst, host, nbytes, slot_off, lens_off,
                                     to_device_raw(k, "bf16", DEV),
                                     to_device_raw(v, "bf16", DEV), out,
                                     to_device_raw(q, "bf16", DEV), b.k_dev, b.v_dev, b.tab_dev,
                                     b.nb, b.h_kv, int(b.lens.max()), b.sm, KS, VS,
                                     ws) == pa.PA_OK
            torch.cuda.synchronize()
            ref, _ = b.oracle_step(slots, k, v, q)
            assert_close(out_to_f64(to_host_raw(out, "bf16"), "bf16"), ref, "bf16",
                         f"one poll, iteration {it}")
            assert np.array_equal(dst.cpu().numpy(), host.numpy())
            assert int(ws[:64].view(torch.int32)[:3].abs().sum()) == 0
    finally:
        assert pa.pa_decode_step_set_spin_limit(65536) == pa.PA_OK


def test_decode_step_full_batch_wide_groups():
    """The largest batch one launch takes (2048 sequences, lengths kept in
    LDS) with 16 query heads per KV head and d = 64: short contexts from
    empty up, two iterations, against the oracle."""
    rng = np.random.default_rng(5600)
    lengths = rng.integers(0, 48, size=2048)
    lengths[:4] = [0, 15, 16, 47]
    b = StepBatch(5601, lengths.tolist(), 32, 2, 64, "bf16", steps=2, extra_blocks=4)
    ws = decode_workspace(b.S, b.h_q, b.h_kv, 64, int(b.lengths.max()) + 2, DEV)
    for it in range(2):
        slots, k, v, q = b.next_tokens()
        host, slot_off, lens_off, nbytes = _meta(b.S, slots, b.lens, pad=1)
        dst = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
        out = torch.full((b.S, b.h_q, 64), SENTINEL, dtype=torch.bfloat16, device=DEV)
        say(f"[decode step] 2048 sequences, 32/2 heads, d64, iteration {it}")
        assert pa.pa_decode_step(None, dst, host, nbytes, slot_off, lens_off,
                                 to_device_raw(k, "bf16", DEV), to_device_raw(v, "bf16", DEV),
                                 out, to_device_raw(q, "bf16", DEV), b.k_dev, b.v_dev, b.tab_dev,
                                 b.nb, b.h_kv, int(b.lens.max()), b.sm, KS, VS, ws) == pa.PA_OK
        torch.cuda.synchronize()
        ref, tables = b.oracle_step(slots, k, v, q)
        assert_close(out_to_f64(to_host_raw(out, "bf16"), "bf16"), ref, "bf16",
                     f"2048 sequences, iteration {it}")
        got_t = b.tab_dev.cpu().numpy()
        for s_ in range(b.S):
            n = _blocks(b.lens[s_])
            assert np.array_equal(got_t[s_, :n], tables[s_, :n]), (it, s_)
