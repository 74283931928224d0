"""Number formats of the oracle (test infrastructure only).

The pages speak of storing keys and values in an 8-bit cache to halve the
memory of a 16-bit one (ultralytics.com glossary "PagedAttention", section
"Related techniques", FP8 cache quantization).  The 8-bit format used here is
OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals m * 2^-9, no infinities, S.1111.111 is NaN, largest finite 448.

Encoding reading (the pages are silent): ``y = fp32(x) / fp32(scale)`` with
IEEE single-precision division, then round to the nearest E4M3 value with ties
to the even mantissa, saturating at +-448; NaN encodes as 0x7F; the sign bit of
y is kept (so -0 and negative values that round to zero encode as 0x80).

bfloat16 values are carried as raw 16-bit patterns: the top half of an IEEE
binary32 word.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_value(code: int) -> float:
    """Value of one E4M3FN code, straight from the format definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return float("nan")
    if exponent == 0:
        return sign * mantissa * 2.0 ** -9            # subnormal: (m / 8) * 2^(1 - 7)
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# magnitudes of codes 0x00 .. 0x7E, strictly increasing
_MAGNITUDES = E4M3_TABLE[:0x7F]


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes -> float64 (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_f32(y: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3FN codes: nearest, ties to even mantissa, saturating.

    The candidates are the 127 finite magnitudes in code order; of the two that
    bracket |y| the nearer wins, and on an exact tie the one with an even code
    (even mantissa bit).  Distances are taken in float64, which is exact at every
    tie (a midpoint of two E4M3 values has at most 5 significant bits) and
    cannot flip a comparison elsewhere (|y| differs from a midpoint by at least
    one float32 ulp, far above float64 rounding).
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    hi = np.searchsorted(_MAGNITUDES, a, side="left")      # first magnitude >= |y|
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _MAGNITUDES[lo]
    d_hi = _MAGNITUDES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a > E4M3_MAX, 0x7E, code)               # saturate (incl. +-inf)
    code = code.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << np.uint8(7))
    code = np.where(np.isnan(y), np.uint8(0x7F), code)
    return code.astype(np.uint8)


def e4m3_quantize(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Encode values for an fp8 cache: ``y = x / scale`` in IEEE float32, then E4M3FN."""
    y = np.asarray(x_f32, dtype=np.float32) / np.float32(scale)
    return e4m3_encode_f32(y)
