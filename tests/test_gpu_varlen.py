"""GPU: pa_attend_varlen -- the decode rows and the prefill slices of one
iteration in a single launch -- against the oracle, and against the separate
pa_decode + pa_prefill_chunk launches.

LESSON "What the scheduler looks like": one call runs the iteration's whole
mixed batch; "Chunked prefill": a slice's queries attend causally to their
prompt's earlier positions and their own.  A decode row is the special case
of a slice of one query at the sequence's last position, so the oracle for
the whole batch is oracle/attention.py's prefill_chunk over every sequence
(the decode rows as one-query slices).  The cases reach the launch's own
machinery: decode contexts cut into several chunks (merged in-kernel by the
last chunk to finish), prefill key ranges split over work-groups (merged by
the last split), empty slices, a batch of only one kind, and repeated calls
that must leave the work counters zero."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_host_amd as pa
from paged_kv_cache_host_amd.engine import varlen_buffers
from tests.gate import assert_close
from tests.parity import out_to_f64
from tests.varlen_parity import Batch, mixed_batch, oracle_varlen as _oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = {
    # decode contexts across block edges and past 2048 tokens (several
    # chunks: merged in-kernel), slices of two prompts with a split key
    # range (max_prefill_len 2900 -> two splits)
    "bf16-16q2kv-d128": dict(decode_lens=[1, 15, 16, 17, 100, 2049, 5000, 700],
                             prompts=[2900, 333],
                             slices=[(0, 2600, 300), (1, 0, 128), (1, 128, 100), (1, 228, 1)]),
    "fp8-16q2kv-d128": dict(decode_lens=[33, 4100, 64, 1], prompts=[2100, 97],
                            slices=[(0, 1900, 200), (1, 0, 97)], cache_dtype="fp8"),
    "bf16-8q1kv-d64": dict(decode_lens=[5, 3000, 47], prompts=[1500, 40],
                           slices=[(0, 1000, 500), (1, 0, 40)], h_q=8, h_kv=1, d=64),
    "bf16-32q2kv-d128": dict(decode_lens=[260, 2300], prompts=[1200],
                             slices=[(0, 1100, 100)], h_q=32, h_kv=2),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_varlen_against_oracle(case):
    c = dict(CASES[case])
    w, n_dec = mixed_batch(f"varlen-{case}", 4100 + len(case), **c)
    say(f"[varlen vs oracle] {case}: {n_dec} decode rows, slices {w.slices[n_dec:]}")
    b = Batch(w, n_dec)
    got, (counters, _) = b.fused()
    ref = _oracle(w)
    err = assert_close(out_to_f64(got, w.q_dtype), ref, w.cache_dtype, f"varlen {case}")
    say(f"  max|d| = {err:.3g}")
    assert int(counters.abs().sum()) == 0, "the launch left its work counters nonzero"


@pytest.mark.parametrize("case", sorted(CASES))
def test_varlen_equals_separate_launches(case):
    """Same splits as the separate launches: the same bits."""
    c = dict(CASES[case])
    w, n_dec = mixed_batch(f"varlen-{case}", 4200 + len(case), **c)
    say(f"[varlen vs separate launches] {case}")
    b = Batch(w, n_dec)
    got, _ = b.fused()
    sep = b.separate()
    assert got.shape == sep.shape
    diff = np.flatnonzero(got.reshape(-1) != sep.reshape(-1))
    assert diff.size == 0, f"{diff.size} outputs differ from the separate launches"


def test_varlen_one_kind_and_empty_slices():
    """Only decode rows; only prefill slices (one of them empty); and an
    empty slice among decode rows."""
    cases = [
        ("decode only", dict(decode_lens=[3, 2500, 16, 4097], prompts=[], slices=[])),
        ("prefill only", dict(decode_lens=[], prompts=[600, 50],
                              slices=[(0, 0, 256), (0, 256, 0), (1, 0, 50), (0, 256, 344)])),
        ("decode + empty slice", dict(decode_lens=[40, 1], prompts=[64],
                                      slices=[(0, 10, 0)])),
    ]
    for i, (what, c) in enumerate(cases):
        w, n_dec = mixed_batch(f"varlen-{what}", 4300 + i, **c)
        say(f"[varlen] {what}")
        b = Batch(w, n_dec)
        got, (counters, _) = b.fused()
        ref = _oracle(w)
        if len(b.rows):
            assert_close(out_to_f64(got, w.q_dtype), ref, w.cache_dtype, f"varlen {what}")
        assert int(counters.abs().sum()) == 0


def test_varlen_buffers_serve_smaller_calls():
    """Counters and workspace sized for the largest call serve a sequence of
    calls with fewer decode rows, fewer and shorter slices and shorter
    contexts (where the prefill range splits more ways), in either order."""
    big_c = dict(decode_lens=[2100, 5000, 70, 9, 3000, 16], prompts=[3000, 2000],
                 slices=[(0, 2488, 512), (1, 1500, 500)])
    w, n_dec = mixed_batch("varlen-big", 4400, **big_c)
    big = Batch(w, n_dec)
    bufs = varlen_buffers(n_dec, 2, w.h_q, w.h_kv, w.d, big.max_q, big.max_dec, big.max_pf, DEV)
    smaller = [
        dict(decode_lens=[5000, 30], prompts=[2600], slices=[(0, 2560, 40)]),
        dict(decode_lens=[2049], prompts=[1100, 900], slices=[(0, 1000, 100), (1, 0, 64)]),
    ]
    calls = [(big, w)]
    for i, c in enumerate(smaller):
        ws_, nd_ = mixed_batch(f"varlen-small{i}", 4410 + i, **c)
        calls.append((Batch(ws_, nd_), ws_))
    for rep in range(2):
        for i, (bt, wt) in enumerate(calls if rep == 0 else calls[::-1]):
            say(f"[varlen shared buffers] call {i} rep {rep}")
            got, _ = bt.fused(bufs)
            assert_close(out_to_f64(got, wt.q_dtype), _oracle(wt), wt.cache_dtype,
                         f"shared buffers call {i} rep {rep}")
            assert int(bufs[0].abs().sum()) == 0


def test_varlen_rejects_bad_arguments():
    """Argument errors come back as statuses before any launch (real device
    buffers throughout)."""
    w, n_dec = mixed_batch("varlen-args", 4500, decode_lens=[20], prompts=[64],
                           slices=[(0, 0, 64)])
    b = Batch(w, n_dec)
    counters, ws = varlen_buffers(1, 1, w.h_q, w.h_kv, w.d, 64, 20, 64, DEV)
    out = torch.zeros((len(b.rows), w.h_q, w.d), dtype=torch.bfloat16, device=DEV)

    def call(**kw):
        a = dict(n_decode=1, max_q_len=64, max_decode_len=20, max_prefill_len=64,
                 counters=counters, ws=ws)
        a.update(kw)
        nd = min(a["n_decode"], 2)
        return pa.pa_attend_varlen(None, out, b.q, b.d_cu, b.d_lens, a["n_decode"], b.kv.k,
                                   b.kv.v, b.tables[:nd], b.tables[nd:], w.num_blocks, w.h_kv,
                                   a["max_q_len"],
                                   a["max_decode_len"], a["max_prefill_len"], w.sm_scale,
                                   counters=a["counters"], ws=a["ws"])

    assert call(counters=counters[:1]) == pa.PA_ERR_WORKSPACE
    assert call(counters=None) == pa.PA_ERR_WORKSPACE
    assert call(max_prefill_len=32) == pa.PA_ERR_INVALID          # < max_q_len
    assert call(max_decode_len=16 * b.max_blocks + 1) == pa.PA_ERR_INVALID
    with pytest.raises(pa.PaError):
        call(n_decode=3)                                          # more than the sequences
    assert call() == pa.PA_OK
    torch.cuda.synchronize()
    assert int(counters.abs().sum()) == 0


def test_partial_tail_tile_is_stable_after_idle_gaps():
    """The last 64-key tile of a position tile's key range is partial (here
    28 valid keys of 64) and the V of its missing keys is cleared in LDS.
    That clearing must not overlap another wave still storing its piece of
    the same tile: the rows that see the last valid keys would otherwise
    read an older tile's values for them.  A slow global load (cold caches
    after the GPU sat idle) is what lets one wave fall behind, so the
    calls here are spaced by idle gaps, and every result must equal the
    first bit for bit (and the oracle)."""
    import time
    w, n_dec = mixed_batch("varlen-tail", 4600, decode_lens=[2100, 5000, 3000],
                           prompts=[3000, 2000], slices=[(0, 2488, 512), (1, 1500, 500)])
    b = Batch(w, n_dec)
    first_f, bufs = b.fused()
    first_s = b.separate()
    assert np.array_equal(first_f, first_s)
    assert_close(out_to_f64(first_f, w.q_dtype), _oracle(w), w.cache_dtype, "partial tail tile")
    rng = np.random.default_rng(11)
    for i in range(10):
        time.sleep(1.2 * rng.random())
        got_f, _ = b.fused(bufs)
        time.sleep(1.2 * rng.random())
        got_s = b.separate()
        for what, got, ref in (("fused", got_f, first_f), ("separate", got_s, first_s)):
            dif = got != ref
            if dif.any():
                rows = np.where(dif.any(axis=(1, 2)))[0]
                raise AssertionError(f"{what} call {i}: {int(dif.sum())} outputs changed, rows "
                                     f"{rows[:8].tolist()}")
