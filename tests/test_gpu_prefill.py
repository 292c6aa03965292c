"""GPU parity: pa_prefill_chunk (causal slices against the paged prefix)
against the oracle, through the C ABI."""
import sys

import numpy as np
import pytest

import workloads
from tests.parity import assert_close, out_to_f64
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


def test_slices_f32():
    w = workloads.prefill_workload("f32", 530, prompt_len=150, chunks=[64, 86], h_q=4, h_kv=4, d=64,
                                   dtype="f32", cache_dtype="f32")
    _check(w, "f32")
