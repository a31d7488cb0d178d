"""bfloat16 round-to-nearest-even, taken directly from fp64.

The epilogue of the method converts the fp32 accumulator to bf16 and writes
it back (Lesson 13, Fig. 13-1 "epilogue only converts and stores"; Fig. 13-2).
The pages do not name the rounding mode; the reading taken here is IEEE
round-to-nearest-even.  The oracle's accumulator is fp64, and it is rounded to
bf16 in ONE step (no fp32 intermediate, which would round twice).

bf16 = 1 sign bit, 8 exponent bits (bias 127, same range as fp32), 7 mantissa
bits; subnormals go down to 2^-133.
"""

import numpy as np

_BF16_MANT = 7
_BF16_MIN_NORMAL_EXP = -126
_BF16_MAX_EXP = 127


def _round_bf16_f64(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp64 value of the nearest bf16 (ties to even); +-inf on overflow."""
    x = np.asarray(x, dtype=np.float64)
    v = np.abs(x)
    finite = np.isfinite(v)
    vv = np.where(finite, v, 0.0)
    _, ex = np.frexp(vv)  # floor(log2 v) = ex - 1 for v > 0
    e = np.maximum(ex - 1, _BF16_MIN_NORMAL_EXP)
    q = np.ldexp(1.0, e - _BF16_MANT)  # grid spacing inside the binade
    n = np.rint(vv / q)  # exact rescale, then ties-to-even on the integer
    r = n * q
    r = np.where(r >= 2.0 ** (_BF16_MAX_EXP + 1), np.inf, r)
    r = np.where(finite, r, v)  # inf stays inf, nan stays nan
    return np.copysign(r, x)


def bf16_rne_bits(x) -> np.ndarray:
    """fp64 (or fp32) values -> uint16 bf16 bit patterns, round-to-nearest-even."""
    r = _round_bf16_f64(x)
    # every bf16 value is exactly an fp32 value, so this cast is exact
    r32 = r.astype(np.float32)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(r)
    # canonical quiet NaN keeping the sign
    bits = np.where(nan, (np.signbit(r).astype(np.uint16) << 15) | np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
