"""GPU: pa_decode_noalloc, the decode entry point that allocates nothing
(its workspace is the library's per-device scratch array), against
pa_decode with a caller workspace on the same inputs, and against the
oracle, through the C ABI: two calls in a row, the second smaller, and a
call beyond the array's limit refused before anything is launched."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_host_amd._pa as pa
import workloads
from paged_kv_cache_host_amd.engine import to_device_raw, to_host_raw
from tests.parity import assert_close, filled, hip_decode_run, oracle_decode_run, out_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _workload(lengths, h_q, h_kv, d, cache_dtype, seed):
    lengths = np.asarray(lengths, dtype=np.int64)
    return workloads.decode_workload(
        f"noalloc-{cache_dtype}-{h_q}q{h_kv}kv-d{d}", seed, lambda rng: lengths, h_q, h_kv, d,
        "bf16", cache_dtype, lambda L: workloads.blocks_needed(L) + 9, q_dtype="bf16")


def _noalloc_against_decode(w, oracle_seqs):
    """pa_decode (caller workspace, via the parity runner) and then
    pa_decode_noalloc over the same cache, tables and queries: the outputs
    must be identical bit for bit (same kernels, same work items), and
    within tolerance of the oracle."""
    say(f"[noalloc] {w.name} S={w.num_seqs} maxL={int(w.lengths.max())}")
    hip = hip_decode_run(w, DEV)
    kv = hip["kv"]
    t_d = torch.from_numpy(hip["tables"]).to(DEV)
    l_d = torch.from_numpy(hip["lens"]).to(DEV)
    q = to_device_raw(w.q, "bf16", DEV)
    out = filled((w.num_seqs, w.h_q, w.d), torch.bfloat16, DEV)
    st = pa.pa_decode_noalloc(None, out, q, kv.k, kv.v, t_d, l_d, w.num_blocks, w.h_kv,
                              int(w.lengths.max()), w.sm_scale, w.k_scale, w.v_scale)
    assert st == pa.PA_OK, pa.pa_last_error()
    torch.cuda.synchronize()
    got_raw = to_host_raw(out, "bf16")
    assert np.array_equal(got_raw, hip["outs"][0]), "pa_decode_noalloc differs from pa_decode"
    ref = oracle_decode_run(w, seqs=oracle_seqs)
    got = out_to_f64(got_raw, "bf16")
    # sampled rows against the oracle; every row finite and written
    err = assert_close(got, ref["out"], w.cache_dtype, w.name)
    say(f"    identical to pa_decode; oracle max|d| = {err:.3g}")
    kv.close()


def test_noalloc_decode_two_calls_second_smaller():
    # first call: contexts spanning two and three 2048-token items, so that
    # split partials go through the scratch array and the merge kernel
    rng = np.random.default_rng(7001)
    long = [2047, 2048, 2049, 4097, 5000, 6100]
    lengths = np.concatenate([long, rng.integers(1, 400, 18)])
    w1 = _workload(lengths, 64, 8, 128, "bf16", seed=7002)
    _noalloc_against_decode(w1, list(range(len(long))) + [len(long), len(lengths) - 1])
    # second call on the same array: fewer sequences, shorter contexts, fp8
    w2 = _workload([1, 17, 300, 2100, 2600], 16, 2, 64, "fp8", seed=7003)
    _noalloc_against_decode(w2, list(range(5)))


def test_noalloc_refuses_calls_beyond_its_array():
    """128 sequences x 64 query heads x D 128 at up to 32768 tokens need
    68 MB of split partials, above the 64 MiB array: PA_ERR_WORKSPACE, and
    nothing launched (every buffer is real and sized for the call; all
    contexts are one token, so even a launch would write no partials)."""
    S, h_q, h_kv, d, nb = 128, 64, 8, 128, 16
    q = torch.zeros((S, h_q, d), dtype=torch.bfloat16, device=DEV)
    out = filled((S, h_q, d), torch.bfloat16, DEV)
    kc = torch.zeros((nb, h_kv, d // 8, 16, 8), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((nb, h_kv, d, 16), dtype=torch.bfloat16, device=DEV)
    tables = torch.zeros((S, 2048), dtype=torch.int32, device=DEV)
    lens = torch.ones(S, dtype=torch.int32, device=DEV)
    need = pa.pa_decode_workspace_bytes(S, h_q, h_kv, d, 32768)
    assert need > (64 << 20)
    st = pa.pa_decode_noalloc(None, out, q, kc, vc, tables, lens, nb, h_kv, 32768,
                              d ** -0.5)
    assert st == pa.PA_ERR_WORKSPACE
    assert "pa_decode_noalloc" in pa.pa_last_error()
    # the same call within the limit (16384 tokens) runs
    assert pa.pa_decode_workspace_bytes(S, h_q, h_kv, d, 16384) < (64 << 20)
    assert pa.pa_decode_noalloc(None, out, q, kc, vc, tables, lens, nb, h_kv, 16384,
                                d ** -0.5) == pa.PA_OK
    torch.cuda.synchronize()
    # every context is one zero-valued token: the output is that V row
    assert (out.float() == 0).all()
