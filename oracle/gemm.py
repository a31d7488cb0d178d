"""Block-scaled FP8 GEMM D = A . B^T -> bf16, plain and slow, in fp64.

Definition (Lesson 13, Fig. 13-1 closed-form equation, written for the NT
layout of the deep-dive blog, section 3, where B is stored [N, K]):

    D[i, j] = sum_g  alpha[i, g] * beta[j // 128, g] * sum_{k < 128} A[i, 128g + k] * B[j, 128g + k]

with A, B the decoded e4m3 values, alpha the 1x128 activation scales and beta
the 128x128 weight scales.  The method forms each 128-wide K block's partial
product, multiplies it by alpha*beta and adds it into a separate accumulator
once per K block, K blocks in ascending order (Fig. 13-1, Fig. 13-2 and the
Q1 answer); the epilogue only converts to bf16.

Exactness of the fp64 evaluation below:
* every e4m3 value is an integer multiple of 2^-9 with magnitude <= 448, so
  every product a*b is a multiple of 2^-18 and every partial sum of <= 128
  products is a multiple of 2^-18 of magnitude <= 128 * 448^2 < 2^25: it
  needs at most 43 significant bits and is EXACT in fp64 for any summation
  order (so a BLAS matmul is a valid primitive for the partial product);
* alpha*beta of two fp32 numbers needs 48 bits: exact in fp64;
* the scaled partial and the running sum are rounded once each in fp64,
  relative error ~1e-16 per K block.
The final bf16 rounding is round-to-nearest-even taken directly from fp64.

Accumulating form ("DeepGEMM architecture deep dive", section 3: every GEMM
of the library is D = C + A @ B, the NT one D = C + A @ B^T): with an fp32
input C the output is fp32, D = fl32(C + accumulator), rounded once
(round-to-nearest-even) from the fp64 sum.

Grouped forms (Lesson 13, Fig. 13-3 and the Q3 answer; deep-dive blog,
section 3 table): every expert shares N and K.
* contiguous: rows of all experts are concatenated; row i belongs to expert
  m_indices[i]; rows whose index is outside [0, G) are padding and are left
  untouched in D;
* masked: expert g owns a fixed-capacity block of max_m rows of A and D; only
  its first masked_m[g] rows are computed (clamped to [0, max_m]); every other
  row of D is left untouched.
"""

import numpy as np

from .e4m3 import decode_e4m3
from .bf16 import bf16_rne_bits


def gemm_nt_acc(a_codes, sfa, b_codes, sfb) -> np.ndarray:
    """fp64 accumulator of the promoted GEMM (before the bf16 epilogue).

    a_codes: uint8 [M, K]; sfa: fp32 [K/128, M] (MN-major)
    b_codes: uint8 [N, K]; sfb: fp32 [ceil(N/128), K/128]
    returns fp64 [M, N]
    """
    a = decode_e4m3(a_codes)
    b = decode_e4m3(b_codes)
    M, K = a.shape
    N, Kb = b.shape
    if K != Kb or K % 128:
        raise ValueError("K mismatch or K not a multiple of 128")
    sfa = np.asarray(sfa, dtype=np.float32).astype(np.float64)
    sfb = np.asarray(sfb, dtype=np.float32).astype(np.float64)
    if sfa.shape != (K // 128, M) or sfb.shape != ((N + 127) // 128, K // 128):
        raise ValueError("scale tensor shape mismatch")
    col_block = np.arange(N) // 128
    acc = np.zeros((M, N), dtype=np.float64)
    for g in range(K // 128):
        ks = slice(128 * g, 128 * g + 128)
        partial = a[:, ks] @ b[:, ks].T  # exact (see module docstring)
        scale = sfa[g][:, None] * sfb[col_block, g][None, :]  # exact
        acc += scale * partial
    return acc


def gemm_nt(a_codes, sfa, b_codes, sfb) -> np.ndarray:
    """bf16 bits (uint16 [M, N]) of D = A . B^T with per-128-K promotion."""
    return bf16_rne_bits(gemm_nt_acc(a_codes, sfa, b_codes, sfb))


def grouped_contiguous(a_codes, sfa, b_codes, sfb, m_indices, d_init) -> np.ndarray:
    """M-grouped contiguous layout.

    a_codes: uint8 [M_total, K]; sfa: fp32 [K/128, M_total]
    b_codes: uint8 [G, N, K];    sfb: fp32 [G, ceil(N/128), K/128]
    m_indices: int32 [M_total]; d_init: uint16 [M_total, N] (prior contents of D)
    returns uint16 [M_total, N]: rows with a valid expert index recomputed,
    every other row equal to d_init.
    """
    m_indices = np.asarray(m_indices, dtype=np.int64)
    G = b_codes.shape[0]
    d = np.array(d_init, dtype=np.uint16, copy=True)
    for e in range(G):
        rows = np.nonzero(m_indices == e)[0]
        if rows.size == 0:
            continue
        d[rows] = gemm_nt(a_codes[rows], sfa[:, rows], b_codes[e], sfb[e])
    return d


def grouped_masked(a_codes, sfa, b_codes, sfb, masked_m, d_init) -> np.ndarray:
    """M-grouped masked layout.

    a_codes: uint8 [G, max_m, K]; sfa: fp32 [G, K/128, max_m]
    b_codes: uint8 [G, N, K];     sfb: fp32 [G, ceil(N/128), K/128]
    masked_m: int32 [G]; d_init: uint16 [G, max_m, N]
    returns uint16 [G, max_m, N]: the first clamp(masked_m[g], 0, max_m) rows of
    each expert recomputed, every other row equal to d_init.
    """
    G, max_m, _ = a_codes.shape
    d = np.array(d_init, dtype=np.uint16, copy=True)
    for g in range(G):
        m = int(min(max(int(masked_m[g]), 0), max_m))
        if m == 0:
            continue
        d[g, :m] = gemm_nt(a_codes[g, :m], sfa[g][:, :m], b_codes[g], sfb[g])
    return d


def gemm_nt_c(a_codes, sfa, b_codes, sfb, c) -> np.ndarray:
    """fp32 [M, N] of D = C + A . B^T (C fp32 [M, N]; None means zero), one
    round-to-nearest-even from fp64 (numpy's fp64 -> fp32 cast rounds to
    nearest even)."""
    acc = gemm_nt_acc(a_codes, sfa, b_codes, sfb)
    if c is not None:
        acc = acc + np.asarray(c, dtype=np.float32).astype(np.float64)
    return acc.astype(np.float32)
