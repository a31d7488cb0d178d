"""Seeded synthetic inputs shaped like DeepSeek-V3 FP8 GEMM workloads.

This module is shared by the tests, the benchmark and the smoke check, and by
both sides of every parity check: it draws fp32 sources, expert row counts and
index arrays, and arranges rows into the grouped layouts.  It holds none of
the method's arithmetic (no quantisation, no GEMM): callers quantise the fp32
sources with the library (GPU) or with the CPU oracle.

Recipe (numpy PCG64, ``numpy.random.default_rng(seed)``), draws in this order:
1. expert row counts -- contiguous: G integers uniform on [1, 8192];
   masked: G integers uniform on [0, max_m];
2. activations A: R x K standard normal fp32 (R = valid rows), then a uniform
   [0, 1) fp32 draw of the same shape; entries where it is < 1e-3 are
   multiplied by 20 (0.1% outliers);
3. weights B: (G*N) x K standard normal fp32 times fp32(1/sqrt(K)), i.e.
   N(0, 1/K).
K-grouped (weight-gradient) inputs: G token counts uniform on [0, max_tokens],
each segment padded to a multiple of 128 positions; A (the output gradient,
transposed) M x K and B (the layer input, transposed) N x K drawn as
activations for the valid positions, zero in the padding.
The pages benchmark "all DeepSeek-V3/R1 inference shapes" on H800 without
listing them (the chart was not preserved), so these generators stand in for
those shapes; no dataset or trained weight is involved.
"""

import math

import numpy as np

M_ALIGN = 128  # per-expert segment alignment of the contiguous layout
TRAP_CODE = 0x7F  # e4m3 NaN: written into padding / masked-off rows of A
TRAP_F32 = np.float32(np.nan)  # written into their activation scales
SENTINEL_BF16 = 0xFFFF  # bf16 NaN pattern prefilled into D

# (M, N, K) of the dense sweep: M outer, (N, K) inner, seeds 100 + index.
SWEEP_M = (64, 128, 4096)
SWEEP_NK = ((2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048))


def sweep_shapes():
    out = []
    s = 0
    for m in SWEEP_M:
        for n, k in SWEEP_NK:
            out.append(dict(M=m, N=n, K=k, seed=100 + s))
            s += 1
    return out


CONFIGS = {
    "dense_small": [dict(M=64, N=2112, K=7168, seed=0)],
    "dense_sweep": sweep_shapes(),
    "dense_large": [dict(M=4096, N=7168, K=16384, seed=200)],
    "contiguous": [dict(G=8, N=4096, K=7168, seed=300), dict(G=8, N=7168, K=2048, seed=301)],
    "masked": [dict(G=32, max_m=256, N=4096, K=7168, seed=400), dict(G=32, max_m=256, N=7168, K=2048, seed=401)],
    # decode-sized masked calls: at most 128 tokens per expert
    "masked_decode": [dict(G=32, max_m=128, N=4096, K=7168, seed=402), dict(G=32, max_m=128, N=7168, K=2048, seed=403)],
    # weight gradients of 8 local experts' up (4096 x 7168) and down (7168 x 2048) projections
    "k_grouped": [dict(G=8, M=4096, N=7168, seed=500), dict(G=8, M=7168, N=2048, seed=501)],
}


def _activations(rng, rows: int, k: int) -> np.ndarray:
    a = rng.standard_normal((rows, k), dtype=np.float32)
    outlier = rng.random((rows, k), dtype=np.float32) < np.float32(1e-3)
    a[outlier] *= np.float32(20.0)
    return a


def _weights(rng, rows: int, k: int) -> np.ndarray:
    b = rng.standard_normal((rows, k), dtype=np.float32)
    b *= np.float32(1.0 / math.sqrt(k))
    return b


def dense(M: int, N: int, K: int, seed: int):
    """fp32 A [M, K] and B [N, K]."""
    rng = np.random.default_rng(seed)
    a = _activations(rng, M, K)
    b = _weights(rng, N, K)
    return a, b


def contiguous(G: int, N: int, K: int, seed: int, max_tokens: int = 8192, counts=None):
    """M-grouped contiguous workload.

    Returns dict with
      counts    int64 [G]        valid rows per expert
      m_indices int32 [M_total]  expert of each row, -1 on padding rows
      rows      int64 [R]        position of each valid row in the padded layout
      a         fp32 [R, K]      valid rows only, expert-major order
      b         fp32 [G, N, K]
    Each expert's segment is padded to a multiple of M_ALIGN rows.
    """
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = rng.integers(1, max_tokens + 1, G)
    counts = np.asarray(counts, dtype=np.int64)
    padded = (counts + M_ALIGN - 1) // M_ALIGN * M_ALIGN
    m_total = int(padded.sum())
    m_indices = np.full(m_total, -1, dtype=np.int32)
    rows = []
    start = 0
    for e in range(G):
        c = int(counts[e])
        m_indices[start:start + c] = e
        rows.append(np.arange(start, start + c, dtype=np.int64))
        start += int(padded[e])
    rows = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    a = _activations(rng, rows.size, K)
    b = _weights(rng, G * N, K).reshape(G, N, K)
    return dict(counts=counts, m_indices=m_indices, rows=rows, a=a, b=b, m_total=m_total)


def masked(G: int, max_m: int, N: int, K: int, seed: int, masked_m=None):
    """M-grouped masked workload.

    Returns dict with
      masked_m int32 [G]       valid rows per expert (first masked_m[g] rows)
      rows     int64 [R]       flat row index g*max_m + r of each valid row
      a        fp32 [R, K]     valid rows only, expert-major order
      b        fp32 [G, N, K]
    """
    rng = np.random.default_rng(seed)
    if masked_m is None:
        masked_m = rng.integers(0, max_m + 1, G)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    rows = np.concatenate(
        [g * max_m + np.arange(min(max(int(masked_m[g]), 0), max_m), dtype=np.int64) for g in range(G)]
    ) if G else np.zeros(0, dtype=np.int64)
    a = _activations(rng, rows.size, K)
    b = _weights(rng, G * N, K).reshape(G, N, K)
    return dict(masked_m=masked_m, rows=rows, a=a, b=b)


def place_rows(codes: np.ndarray, scales: np.ndarray, rows: np.ndarray, total_rows: int):
    """Place quantised valid rows into a padded row layout, trapping the rest.

    codes  uint8 [R, K] and scales fp32 [K/128, R] of the valid rows
    returns uint8 [total_rows, K] with TRAP_CODE on the other rows and
            fp32 [K/128, total_rows] with TRAP_F32 on the other rows.
    """
    K = codes.shape[1]
    out_q = np.full((total_rows, K), TRAP_CODE, dtype=np.uint8)
    out_s = np.full((scales.shape[0], total_rows), TRAP_F32, dtype=np.float32)
    out_q[rows] = codes
    out_s[:, rows] = scales
    return out_q, out_s


def dense_bf16(M: int, N: int, K: int, seed: int):
    """BF16 operands (uint16 bit patterns): A ~ N(0, 1), B ~ N(0, 1/K), drawn in
    fp32 as for the FP8 workloads and cast to bf16 by torch (round to nearest
    even)."""
    import torch

    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    b = rng.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
    cast = lambda x: torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return cast(a), cast(b)


def k_grouped(G: int, M: int, N: int, seed: int, max_tokens: int = 8192, counts=None):
    """K-grouped (weight-gradient) workload.

    Returns dict with
      counts int64 [G]   tokens per expert (0 allowed)
      ks     int32 [G]   segment lengths: counts padded to multiples of 128
      a      fp32 [M, K] output gradient, transposed (tokens along K)
      b      fp32 [N, K] layer input, transposed
    Padding positions of every segment are zero in both operands.
    """
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = rng.integers(0, max_tokens + 1, G)
    counts = np.asarray(counts, dtype=np.int64)
    ks = ((counts + 127) // 128 * 128).astype(np.int32)
    K = int(ks.sum())
    valid = np.zeros(K, dtype=bool)
    lo = 0
    for g in range(G):
        valid[lo:lo + int(counts[g])] = True
        lo += int(ks[g])
    a = np.zeros((M, K), dtype=np.float32)
    b = np.zeros((N, K), dtype=np.float32)
    nv = int(valid.sum())
    a[:, valid] = _activations(rng, M, nv)
    b[:, valid] = _activations(rng, N, nv)
    return dict(counts=counts, ks=ks, a=a, b=b)
