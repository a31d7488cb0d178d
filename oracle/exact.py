"""Exact rational brute force for tiny shapes (pins the fp64 oracle).

Evaluates the closed-form equation of Lesson 13, Fig. 13-1 with Python
Fractions -- no floating point anywhere between the stored inputs and the final
rounding -- and rounds the exact rational result to bf16 with
round-to-nearest-even.  It decodes e4m3 bytes and rounds to bf16 with its own
rational arithmetic, independent of ``e4m3.py`` and ``bf16.py``, so agreement
with ``gemm.py`` checks those modules too.  Pure-Python loops: tiny inputs only.
"""

from fractions import Fraction

import numpy as np


def e4m3_fraction(code: int):
    """Exact value of an e4m3 (OCP E4M3FN) byte as a Fraction, or None for NaN."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return None
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 2 ** 6)
    mag = Fraction(8 + m, 8)
    return s * (mag * 2 ** (e - 7) if e >= 7 else mag / 2 ** (7 - e))


def f32_fraction(v) -> Fraction:
    """Exact value of a finite fp32 number."""
    return Fraction(float(np.float32(v)))


def bf16_bits_from_fraction(x: Fraction) -> int:
    """Round an exact rational to bf16 (ties to even) and return the 16-bit pattern."""
    if x == 0:
        return 0  # exact zero: +0 (sign of zero is not observable from a rational)
    sign = 0x8000 if x < 0 else 0
    v = abs(x)
    # find e with 2^e <= v < 2^(e+1)
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    e = max(e, -126)  # below the smallest normal the spacing stays 2^-133
    q = Fraction(2) ** (e - 7)
    t = v / q
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * q
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80  # overflow to infinity
    # encode r = n * 2^(e-7) as bf16 fields
    if r < Fraction(2) ** -126:
        # subnormal: mantissa = r / 2^-133
        return sign | int(r / Fraction(2) ** -133)
    ee = r.numerator.bit_length() - r.denominator.bit_length()
    while Fraction(2) ** ee > r:
        ee -= 1
    while Fraction(2) ** (ee + 1) <= r:
        ee += 1
    mant = r / Fraction(2) ** ee - 1  # in [0, 1)
    m7 = mant * 128
    assert m7.denominator == 1
    return sign | ((ee + 127) << 7) | int(m7)


def gemm_nt_exact(a_codes, sfa, b_codes, sfb):
    """Exact closed form; returns (Fraction matrix as nested lists, uint16 bf16 bits)."""
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    b_codes = np.asarray(b_codes, dtype=np.uint8)
    M, K = a_codes.shape
    N = b_codes.shape[0]
    A = [[e4m3_fraction(int(c)) for c in row] for row in a_codes]
    B = [[e4m3_fraction(int(c)) for c in row] for row in b_codes]
    out = np.zeros((M, N), dtype=np.uint16)
    exact = []
    for i in range(M):
        row = []
        for j in range(N):
            total = Fraction(0)
            for g in range(K // 128):
                part = sum(A[i][128 * g + k] * B[j][128 * g + k] for k in range(128))
                total += f32_fraction(sfa[g][i]) * f32_fraction(sfb[j // 128][g]) * part
            row.append(total)
            out[i, j] = bf16_bits_from_fraction(total)
        exact.append(row)
    return exact, out


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern, from the format definition
    (1 sign, 8 exponent bits with bias 127, 7 mantissa bits, subnormals)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF, "inf/nan have no rational value"
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def gemm_bf16_nt_exact(a_bits, b_bits):
    """Exact sum of products of bf16 operands, rounded once to bf16 (bits)."""
    a_bits = np.asarray(a_bits, dtype=np.uint16)
    b_bits = np.asarray(b_bits, dtype=np.uint16)
    M, K = a_bits.shape
    N = b_bits.shape[0]
    A = [[bf16_fraction(int(c)) for c in row] for row in a_bits]
    B = [[bf16_fraction(int(c)) for c in row] for row in b_bits]
    out = np.zeros((M, N), dtype=np.uint16)
    for i in range(M):
        for j in range(N):
            out[i, j] = bf16_bits_from_fraction(sum(A[i][k] * B[j][k] for k in range(K)))
    return out


def f32_from_fraction(x: Fraction) -> np.float32:
    """Round an exact rational to fp32 (ties to even); +-inf past the range."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    v = abs(x)
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    e = max(e, -126)  # below the smallest normal the spacing stays 2^-149
    q = Fraction(2) ** (e - 23)
    t = v / q
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * q
    if r >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(r))  # r has <= 24 significant bits: exact in fp64 and fp32


def gemm_nt_c_exact(a_codes, sfa, b_codes, sfb, c):
    """Exact closed form plus C, rounded once to fp32."""
    exact, _ = gemm_nt_exact(a_codes, sfa, b_codes, sfb)
    M, N = len(exact), len(exact[0]) if exact else 0
    out = np.zeros((M, N), dtype=np.float32)
    for i in range(M):
        for j in range(N):
            cc = f32_fraction(c[i][j]) if c is not None else Fraction(0)
            out[i, j] = f32_from_fraction(exact[i][j] + cc)
    return out


def k_grouped_exact(a_codes, sfa, b_codes, sfb, ks, c):
    """Exact K-grouped form: per group, C plus the sum over the group's K
    blocks of alpha[block][row] * beta[block][col] * (exact block partial),
    rounded once to fp32.  Segment bounds are walked here from ks directly."""
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    b_codes = np.asarray(b_codes, dtype=np.uint8)
    M, K = a_codes.shape
    N = b_codes.shape[0]
    A = [[e4m3_fraction(int(v)) for v in row] for row in a_codes]
    B = [[e4m3_fraction(int(v)) for v in row] for row in b_codes]
    G = len(ks)
    out = np.zeros((G, M, N), dtype=np.float32)
    start = 0
    for g in range(G):
        stop = start + int(ks[g])
        for i in range(M):
            for j in range(N):
                total = f32_fraction(c[g][i][j]) if c is not None else Fraction(0)
                for k0 in range(start, stop, 128):
                    part = sum(A[i][k] * B[j][k] for k in range(k0, k0 + 128))
                    total += f32_fraction(sfa[k0 // 128][i]) * f32_fraction(sfb[k0 // 128][j]) * part
                out[g, i, j] = f32_from_fraction(total)
        start = stop
    return out
