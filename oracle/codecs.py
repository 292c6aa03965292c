"""Storage formats of the KV cache, queries and outputs (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The cache of the ARTICLE (§2.2, block manager) is a tensor of a fixed element
type; the workloads here store it as fp32, bf16 or the OCP 8-bit float
"e4m3fn" with a per-tensor fp32 scale.  Each decoder here maps stored bits to
the exact real value they denote (as fp64); each encoder rounds a float32 to
the nearest representable value, ties to the even code.

Definitions used (the formats themselves, not any library):
  bf16     1 sign, 8 exponent, 7 mantissa bits; the top half of an IEEE
           binary32.  Decoding = shift left by 16 and reinterpret.
  e4m3fn   1 sign, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
           field 0 is subnormal: value = m * 2^-9.  Otherwise
           value = (1 + m/8) * 2^(e-7).  No infinities; only the codes with
           all exponent and mantissa bits set (0x7F, 0xFF) are NaN, so the
           largest finite magnitude is 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- bf16 -----


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 codes -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_encode(x) -> np.ndarray:
    """float32 values -> uint16 bf16 codes, round to nearest, ties to even.

    NaN maps to a quiet NaN of the same sign.  The rounding is carried out on
    the binary32 bit pattern: adding 0x7FFF plus the lowest kept bit and
    truncating the low 16 bits is exactly round-half-to-even on the dropped
    half-word (a carry into the exponent yields the next binade, and past the
    largest finite value, infinity, as IEEE rounding does).
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
        r = np.where(nan, sign | np.uint16(0x7FC0), r).astype(np.uint16)
    return r


# -------------------------------------------------------------- e4m3fn -----

E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * m * 2.0 ** -9
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_TABLE = _e4m3_table()

# Non-negative finite codes 0x00..0x7E in increasing value order (the code
# order is already monotone for one sign).
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = E4M3_TABLE[:0x7F]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> exact fp64 values (NaN for 0x7F / 0xFF)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def e4m3_encode_sat(v) -> np.ndarray:
    """float32 values -> e4m3fn codes: nearest finite value, ties to the even
    code (even mantissa), magnitudes above 448 saturate to +-448, NaN -> NaN.

    The sign is kept, so values that round to zero give +0 (0x00) or -0
    (0x80).  Implemented as a nearest-neighbour search over the 127
    non-negative finite values.
    """
    f = np.asarray(v, dtype=np.float32)
    a = np.abs(f.astype(np.float64))
    neg = np.signbit(f)
    nan = np.isnan(f)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_POS_VALS, a, side="left")       # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    d_hi = _POS_VALS[hi] - a
    d_lo = a - _POS_VALS[lo]
    exact = d_hi == 0.0
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    code = np.where(exact, _POS_CODES[hi], np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi]))
    code = np.where(nan, 0x7F, code)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def e4m3_quantize(x_f32, scale_f32) -> np.ndarray:
    """Quantise values into the fp8 cache with a per-tensor scale.

    The stored code is ``e4m3_encode_sat(float32(float32(x) * inv))`` where
    ``inv = float32(1) / float32(scale)`` is one float32 reciprocal computed
    once; the product is a single IEEE binary32 multiply (round to nearest
    even).  Decoding multiplies the code's value by ``scale``.
    """
    inv = np.float32(1.0) / np.float32(scale_f32)
    prod = (np.asarray(x_f32, dtype=np.float32) * inv).astype(np.float32)
    return e4m3_encode_sat(prod)


# -------------------------------------------------------------- helpers ----

DTYPES = ("f32", "bf16", "fp8")


def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage array (float32 / uint16 / uint8) -> exact fp64 values."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_decode(raw)
    if dtype == "fp8":
        return e4m3_decode(raw)
    raise ValueError(dtype)


def storage_numpy_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]
