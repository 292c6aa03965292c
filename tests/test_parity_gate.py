"""The parity gate itself (CPU): it must fail on outputs that are not numbers,
on rows no kernel wrote, and outside the stated tolerances."""
import numpy as np
import pytest
import torch

from tests.gate import SENTINEL, TOL, assert_close


def _pair(seed=0, shape=(6, 4, 8)):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal(shape)
    got = ref + rng.uniform(-1e-3, 1e-3, shape)
    return got, ref


def test_close_values_pass_and_worst_is_finite():
    got, ref = _pair()
    err = assert_close(got, ref, "bf16")
    assert np.isfinite(err) and 0 < err <= 1e-3


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_output_fails(bad):
    got, ref = _pair()
    got[2, 1, 3] = bad
    with pytest.raises(AssertionError, match="not finite"):
        assert_close(got, ref, "bf16")


def test_all_nan_output_fails():
    _, ref = _pair()
    with pytest.raises(AssertionError):
        assert_close(np.full(ref.shape, np.nan), ref, "bf16")


def test_non_finite_output_fails_where_the_oracle_computed_nothing():
    # sampled comparisons: the oracle leaves unselected rows NaN, the GPU
    # output must still be finite there
    got, ref = _pair()
    ref[3:] = np.nan
    got[4, 0, 0] = np.nan
    with pytest.raises(AssertionError, match="not finite"):
        assert_close(got, ref, "bf16")


def test_unwritten_row_fails_even_unsampled():
    got, ref = _pair()
    ref[3:] = np.nan
    got[5] = SENTINEL
    with pytest.raises(AssertionError, match="no kernel wrote"):
        assert_close(got, ref, "bf16")


def test_sentinel_is_exact_in_every_output_format():
    for dt in (torch.float32, torch.bfloat16, torch.float16):
        assert float(torch.tensor(SENTINEL, dtype=dt).item()) == SENTINEL
    # and well outside any softmax-weighted mean of the stored values
    assert SENTINEL > 1e3


def test_infinite_reference_fails():
    got, ref = _pair()
    ref[0, 0, 0] = np.inf
    with pytest.raises(AssertionError, match="oracle"):
        assert_close(got, ref, "bf16")


def test_nothing_compared_fails():
    got, ref = _pair()
    with pytest.raises(AssertionError, match="none"):
        assert_close(got, np.full(ref.shape, np.nan), "bf16")


def test_shape_mismatch_fails():
    got, ref = _pair()
    with pytest.raises(AssertionError, match="shape"):
        assert_close(got[:-1], ref, "bf16")


@pytest.mark.parametrize("dt", ["bf16", "fp8", "f32"])
def test_tolerance_edges(dt):
    atol, rtol = TOL[dt]
    ref = np.array([0.0, 1.0, -2.0, 10.0])
    lim = atol + rtol * np.abs(ref)
    assert_close(ref + 0.999 * lim, ref, dt)
    assert_close(ref - 0.999 * lim, ref, dt)
    for i in range(len(ref)):
        got = ref.copy()
        got[i] += 1.001 * lim[i]
        with pytest.raises(AssertionError, match="outside tolerance"):
            assert_close(got, ref, dt)


def test_tolerances_are_the_stated_ones():
    assert TOL["bf16"] == (2e-3, 1e-2)
    assert TOL["fp8"] == (3e-2, 1e-2)
