"""The parity gate: the comparison rule every GPU parity test applies to an
attention output against the oracle's fp64 value.

An output element passes when ``|got - ref| <= atol + rtol * |ref|`` with
(atol, rtol) = (2e-3, 1e-2) for bf16 inputs with fp32 accumulation and
(3e-2, 1e-2) for an fp8 e4m3fn cache; fp32 problems use the bf16 gate.

The gate is strict about values that are not numbers:

* every element of ``got`` must be finite, including the elements the
  oracle did not compute (sampled tests), so a NaN or an infinity produced
  anywhere fails;
* no element of ``got`` may equal ``SENTINEL``: outputs are filled with it
  before a launch, so a row that no work-group writes fails even where the
  oracle has no value to compare with;
* ``ref`` marks the entries the oracle was not asked to compute with NaN
  (its ``pairs``/``rows`` selections); every other ``ref`` entry must be
  finite, and at least one entry must be compared.

Holds no torch and no GPU code, so the CPU suite tests the gate itself.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": (2e-3, 1e-2), "bf16": (2e-3, 1e-2), "fp8": (3e-2, 1e-2)}

# 1.5 * 2^13: exact in fp32, bf16 and fp16, and far outside any softmax-
# weighted mean of the N(0,1) values the workloads store (|v| < 10).
SENTINEL = 12288.0


def assert_close(got, ref, cache_dtype, what=""):
    """Raises AssertionError unless ``got`` passes the gate against ``ref``;
    returns the largest absolute difference over the compared entries (a
    finite number)."""
    atol, rtol = TOL[cache_dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError(f"{what}: shape {got.shape} against the oracle's {ref.shape}")
    bad_num = ~np.isfinite(got)
    if bad_num.any():
        idx = tuple(int(i[0]) for i in np.nonzero(bad_num))
        raise AssertionError(f"{what}: {int(bad_num.sum())} of {got.size} outputs are not finite "
                             f"(first at {idx}: {got[idx]})")
    unwritten = got == SENTINEL
    if unwritten.any():
        idx = tuple(int(i[0]) for i in np.nonzero(unwritten))
        raise AssertionError(f"{what}: {int(unwritten.sum())} outputs still hold the pre-launch "
                             f"fill value (first at {idx}): rows no kernel wrote")
    computed = ~np.isnan(ref)
    if not computed.any():
        raise AssertionError(f"{what}: the oracle computed none of the {ref.size} entries")
    r = ref[computed]
    if not np.isfinite(r).all():
        raise AssertionError(f"{what}: the oracle produced {int((~np.isfinite(r)).sum())} "
                             f"infinite values")
    g = got[computed]
    d = np.abs(g - r)
    lim = atol + rtol * np.abs(r)
    bad = d > lim
    if bad.any():
        i = int(np.argmax(d - lim))
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside tolerance; worst "
                             f"|d|={d[i]:.3g} at ref={r[i]:.4g}, got={g[i]:.4g}")
    return float(d.max())
