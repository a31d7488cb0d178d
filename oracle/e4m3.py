"""FP8 E4M3 (OCP "E4M3FN") decode and encode, written from the format definition.

The pages fix the format by its field split (4 exponent bits, 3 mantissa
bits) and its largest finite magnitude, 448 (Lesson 13, Fig. 13-1 and the
answer to Q1).  That maximum identifies the OCP E4M3FN variant -- exponent
bias 7, no infinities, only the all-ones pattern S.1111.111 is NaN -- and not
the FNUZ variant whose maximum is 240.

Encoding rule (the pages are silent; reading taken here): round to nearest on
the e4m3 grid, subnormals included, ties to the code with an even mantissa;
the sign of zero is kept; magnitudes at or above 448 saturate to +-448 (the
quantiser never produces them: x/alpha <= 448 up to one fp32 ulp).
NaN inputs map to the NaN code with the input's sign.
"""

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7
_MIN_NORMAL_EXP = 1 - _BIAS  # -6
_MANT_BITS = 3


def _decode_one(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        # subnormal: m/8 * 2^(1-bias)
        return sign * (m / 8.0) * 2.0 ** _MIN_NORMAL_EXP
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - _BIAS)


# 256-entry fp64 table built from the definition above.
DECODE_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """uint8 codes (any shape) -> fp64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    return DECODE_TABLE[codes]


def encode_e4m3(x) -> np.ndarray:
    """fp32 (or fp64) values -> uint8 e4m3 codes, round-to-nearest-even.

    Each finite magnitude v is placed in its binade [2^e, 2^(e+1)) with e
    clamped below at the smallest normal exponent (-6, which also covers the
    subnormal range).  The grid spacing there is q = 2^(e-3); n = rint(v / q)
    is exact (v/q is a power-of-two rescaling) and numpy's rint breaks ties
    to even.  Because every binade holds 8 steps, an even n is exactly an
    even mantissa field, so ties-to-even on n is ties-to-even on the code.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    v = np.abs(x)
    nan = np.isnan(v)
    v = np.where(nan, 0.0, v)
    sat = v >= E4M3_MAX
    v = np.where(sat, 0.0, v)

    _, ex = np.frexp(v)  # v = f * 2^ex with f in [0.5, 1); floor(log2 v) = ex - 1
    e = np.maximum(ex - 1, _MIN_NORMAL_EXP)
    q = np.ldexp(1.0, e - _MANT_BITS)
    n = np.rint(v / q)  # integer in [0, 16]
    val = n * q
    # rounding can carry into the next binade (n == 16); recompute fields from val
    val = np.where(sat, E4M3_MAX, val)

    _, ex2 = np.frexp(val)
    is_normal = val >= 2.0 ** _MIN_NORMAL_EXP
    e_unb = np.where(is_normal, ex2 - 1, _MIN_NORMAL_EXP)
    e_field = np.where(is_normal, e_unb + _BIAS, 0)
    mant = np.where(
        is_normal,
        val / np.ldexp(1.0, e_unb) * 8.0 - 8.0,
        val / 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS),
    )
    code = (e_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)
