"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars: quantiser bytes and scales bit-exact; untouched rows bit-exact; GEMM
elements within |d - ref| <= 2^-7 |ref| + 1e-3 rms(ref) with NaN positions
equal; integer inputs with unit scales bit-exact.  Small cases compare every
element; full-size cases run in the benchmark's launch configuration (GPU
quantisers feeding the GEMM) and compare sampled rows/columns that the oracle
computes from its own quantisation of the same fp32 sources, after checking
that the GPU bytes of those rows/blocks equal the oracle's.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import SENTINEL, assert_close, masked_layout

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _np(t):
    torch.cuda.synchronize()
    x = t.cpu().numpy()
    return x.view(np.uint16) if x.dtype == np.int16 else x


def _sentinel(*shape):
    return torch.full(shape, -1, dtype=torch.int16, device=DEV)


def _ws(M, N, K):
    n = dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT, M, N, K, 1)
    return torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV) if n else None


def _gpu_dense(qa, sa, qb, sb, M, N, K, workspace=True):
    D = _sentinel(M, N)
    dg.dg_fp8_gemm_nt(_t(qa), _t(sa), _t(qb), _t(sb), D, _ws(M, N, K) if workspace else None)
    return _np(D)


# ---------------------------------------------------------------- quantisers

# the last two cases have 65576 and 65688 groups: a grid of over 4096
# workgroups whose last one is partly filled
@pytest.mark.parametrize("G,M,K", [(1, 1, 128), (1, 70, 512), (3, 33, 384), (1, 64, 7168), (1, 1171, 7168),
                                   (3, 391, 7168)])
def test_quant_1x128_bit_exact(G, M, K):
    rng = np.random.default_rng(G * 100 + M)
    x = rng.standard_normal((G, M, K), dtype=np.float32) * np.exp2(rng.integers(-30, 30, (G, M, 1))).astype(np.float32)
    x[0, 0, :128] = 0.0  # all-zero group
    x[0, 0, 5] = -0.0
    if K > 128:
        x[0, 0, 128:256] *= np.float32(1e-3)  # codes in the e4m3 subnormal range too
    q = torch.empty((G, M, K), dtype=torch.uint8, device=DEV)
    s = torch.empty((G, K // 128, M), dtype=torch.float32, device=DEV)
    dg.dg_quant_1x128(_t(x), q, s)
    qr, sr = oracle.quant_1x128(x)
    assert np.array_equal(_np(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(_np(q), qr)


def test_quant_1x128_rounding_ties_and_subnormals():
    # each row: amax 448 so alpha = 1 and x/alpha = x exactly; the rest are
    # e4m3 ties, subnormals, signed zeros and values near the saturation edge
    vals = np.array([448, 432, 17, 19, 2.0 ** -10, 3 * 2.0 ** -10, 1.5 * 2.0 ** -9, -1e-4, -0.0, 447.9, 0.0,
                     2.0 ** -6 - 2.0 ** -11, 240, 232, 1.0625, 1.1875], np.float32)
    x = np.zeros((2, 128), np.float32)
    x[0, :vals.size] = vals
    x[1, :vals.size] = -vals
    x[1, 0] = -448
    q = torch.empty((2, 128), dtype=torch.uint8, device=DEV)
    s = torch.empty((1, 2), dtype=torch.float32, device=DEV)
    dg.dg_quant_1x128(_t(x), q, s)
    qr, sr = oracle.quant_1x128(x)
    assert np.all(sr == 1.0) and np.array_equal(_np(s), sr)
    assert np.array_equal(_np(q), qr)


def test_quant_1x128_near_rounding_midpoints():
    # scales other than 1 and values within a few ulps of e4m3 rounding
    # midpoints times the scale: x * (1 / alpha) and fl32(x / alpha) can then
    # fall on different sides of a midpoint, so the kernel must take the exact
    # quotient there to match the oracle's bytes
    rng = np.random.default_rng(11)
    rows = []
    for c in (3.0, 5.0, 0.3, 7e-3, 1.7e5, 1.0 / 3.0):
        amax = np.float32(448.0 * c)
        alpha = np.float32(amax / np.float32(448.0))
        row = [amax]
        while len(row) < 128:
            e = int(rng.integers(-5, 8))
            k = int(rng.integers(0, 8))
            mid = np.float32((1.0 + (2 * k + 1) / 16.0) * 2.0 ** e)  # halfway between two e4m3 codes
            x = np.float32(mid * alpha)
            for j in range(-3, 4):
                v = x
                step = np.float32(np.inf) if j > 0 else np.float32(-np.inf)
                for _ in range(abs(j)):
                    v = np.nextafter(v, step, dtype=np.float32)
                if abs(v) < amax and len(row) < 128:
                    row.append(v if rng.random() < 0.5 else -v)
        rows.append(row)
    x = np.array(rows, np.float32)
    q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    s = torch.empty((1, x.shape[0]), dtype=torch.float32, device=DEV)
    dg.dg_quant_1x128(_t(x), q, s)
    qr, sr = oracle.quant_1x128(x)
    assert np.array_equal(_np(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(_np(q), qr)


def _extreme_groups(rows, seed):
    # one 128-element group per row, amax spread from fp32 subnormals (where
    # alpha is subnormal and 1 / alpha overflows) to the top of the range
    rng = np.random.default_rng(seed)
    amax = np.array([2.0 ** -149, 2.0 ** -140, 2.0 ** -133, 2.0 ** -126, 1e-38, 3e-36, 1.0, 3e30, 1e38, 3.4e38],
                    np.float32)
    x = rng.uniform(-1, 1, (rows, 128)).astype(np.float32) * amax[np.arange(rows) % amax.size, None]
    x[np.arange(rows), rng.integers(0, 128, rows)] = amax[np.arange(rows) % amax.size]
    return x


def test_quant_1x128_extreme_scales():
    x = _extreme_groups(40, 5)
    q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    s = torch.empty((1, x.shape[0]), dtype=torch.float32, device=DEV)
    dg.dg_quant_1x128(_t(x), q, s)
    qr, sr = oracle.quant_1x128(x)
    assert np.array_equal(_np(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(_np(q), qr)


def test_quant_128x128_extreme_scales_and_midpoints():
    # top block row: one block per amax from fp32 subnormals to the top of the
    # range; bottom: alpha = 1/3 and values within a few ulps of e4m3
    # rounding midpoints times alpha
    rng = np.random.default_rng(13)
    amax = np.array([2.0 ** -149, 2.0 ** -140, 2.0 ** -133, 2.0 ** -126, 1e-38, 3e-36, 1.0, 3e30, 1e38, 3.4e38],
                    np.float32)
    top = rng.uniform(-1, 1, (128, 128 * amax.size)).astype(np.float32) * np.repeat(amax, 128)[None]
    top[rng.integers(0, 128, amax.size), np.arange(amax.size) * 128 + 5] = amax
    amid = np.float32(448.0 / 3.0)
    alpha = np.float32(amid / np.float32(448.0))
    mids = ((1.0 + (2 * rng.integers(0, 8, top.shape) + 1) / 16.0) * np.exp2(rng.integers(-5, 7, top.shape)))
    near = (mids.astype(np.float32) * alpha).view(np.int32) + rng.integers(-3, 4, top.shape).astype(np.int32)
    bot = near.view(np.float32) * np.where(rng.random(top.shape) < 0.5, -1, 1).astype(np.float32)
    bot = np.clip(bot, -amid, amid)
    bot[0, ::128] = amid
    x = np.concatenate([top, bot], 0)[None]
    q = torch.empty(x.shape, dtype=torch.uint8, device=DEV)
    s = torch.empty((1, 2, x.shape[2] // 128), dtype=torch.float32, device=DEV)
    dg.dg_quant_128x128(_t(x), q, s)
    qr, sr = oracle.quant_128x128(x)
    assert np.array_equal(_np(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(_np(q), qr)


@pytest.mark.parametrize("G,N,K", [(1, 16, 128), (1, 200, 384), (2, 136, 256), (1, 2112, 1024)])
def test_quant_128x128_bit_exact(G, N, K):
    rng = np.random.default_rng(N + K)
    x = rng.standard_normal((G, N, K), dtype=np.float32) / np.float32(np.sqrt(K))
    x[0, :, :128] = 0.0  # all-zero blocks in the first column block
    q = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    s = torch.empty((G, (N + 127) // 128, K // 128), dtype=torch.float32, device=DEV)
    dg.dg_quant_128x128(_t(x), q, s)
    qr, sr = oracle.quant_128x128(x)
    assert np.array_equal(_np(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(_np(q), qr)


# ---------------------------------------------------------------- dense GEMM

DENSE_SMALL = [(1, 16, 128), (64, 2112, 512), (70, 272, 512), (128, 384, 256), (130, 144, 640), (257, 400, 384),
               (64, 128, 2048),
               # large-tile kernel: K blocks 1..5 exercise every ring-slot tail, ragged M and N
               (256, 128, 128), (300, 272, 256), (512, 384, 384), (1000, 528, 512), (777, 2112, 640), (2048, 256, 1024)]


@pytest.mark.parametrize("M,N,K", DENSE_SMALL)
@pytest.mark.parametrize("workspace", [True, False])
def test_dense_matches_oracle(M, N, K, workspace):
    a32, b32 = workloads.dense(M, N, K, seed=M * 7 + N + K)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    got = _gpu_dense(qa, sa, qb, sb, M, N, K, workspace)
    assert_close(got, oracle.gemm_nt(qa, sa, qb, sb), f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 272, 512), (128, 256, 384), (200, 144, 1024), (1, 16, 256), (512, 400, 640),
                                   (333, 1536, 2048), (2100, 400, 640)])
def test_dense_integer_inputs_bit_exact(M, N, K):
    # integers in [-10, 9] with unit scales: every partial and every fp32 sum is
    # an exact integer below 2^24, so the bf16 result must equal the oracle's bits
    rng = np.random.default_rng(M + N)
    qa = oracle.encode_e4m3(rng.integers(-10, 10, (M, K)).astype(np.float32))
    qb = oracle.encode_e4m3(rng.integers(-10, 10, (N, K)).astype(np.float32))
    sa = np.ones((K // 128, M), np.float32)
    sb = np.ones(((N + 127) // 128, K // 128), np.float32)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    for ws in (True, False):
        assert np.array_equal(_gpu_dense(qa, sa, qb, sb, M, N, K, ws), ref)


def test_dense_power_of_two_scaling_bit_exact():
    M, N, K = 96, 256, 512
    a32, b32 = workloads.dense(M, N, K, seed=5)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    base = _gpu_dense(qa, sa, qb, sb, M, N, K)
    scaled = _gpu_dense(qa, sa * np.float32(4.0), qb, sb * np.float32(0.5), M, N, K)
    assert np.array_equal(oracle.bf16_bits_to_f64(scaled), oracle.bf16_bits_to_f64(base) * 2.0)


def test_dense_deterministic_and_nan_rows_contained():
    M, N, K = 64, 2112, 1024
    a32, b32 = workloads.dense(M, N, K, seed=6)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    qa[5, 300] = 0x7F  # NaN code: poisons row 5 only
    d1 = _gpu_dense(qa, sa, qb, sb, M, N, K)
    d2 = _gpu_dense(qa, sa, qb, sb, M, N, K)
    assert np.array_equal(d1, d2)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    assert_close(d1, ref, "dense with a NaN row")


# skinny kernel (M <= 128): one or many K splits, ragged M and N, splits whose
# block count is not a multiple of the ring depth, and one workspace reused
# across calls (its split counters must come back to zero after every call)
SKINNY = [(1, 2112, 7168), (17, 144, 1024), (64, 2112, 7168), (100, 272, 4096), (128, 2112, 7168),
          (64, 4096, 640), (128, 32768, 512), (33, 24576, 1536), (64, 7168, 2048),
          (100, 7168, 5120)]  # the last: one 128-row tile of 128 columns, K split in 4

# skinny kernel with several row tiles (128 < M <= 2048, few columns or
# short K): 64x64 tiles up to 256 rows, then 64x64, 64x128 or 128x128 tiles,
# with and without a K split, ragged last row tile
SKINNY_MID = [(129, 144, 640), (160, 2112, 7168), (193, 400, 1024), (256, 7168, 2048), (250, 1008, 3072),
              (257, 144, 3072), (400, 2112, 1024), (333, 1536, 7168), (257, 7168, 1024), (333, 4096, 5120),
              (520, 144, 3072), (700, 1536, 1024), (520, 1008, 7168), (777, 2112, 1024), (700, 1536, 5120),
              (2048, 1024, 2048)]


# persistent kernel (M > 2048, or K > 8192): tile counts that leave a partial
# last round, so tail tiles are split along K into pieces (2 to 4, including a
# short last piece), and one whole round, again with one workspace reused
# across calls
PERSISTENT_TAIL = [(200, 144, 9216), (257, 400, 9216), (2100, 272, 1024), (2300, 528, 512), (2300, 384, 640),
                   (2048, 4096, 1536)]


@pytest.mark.parametrize("M,N,K", SKINNY + SKINNY_MID + PERSISTENT_TAIL)
def test_dense_skinny_matches_oracle_with_reused_workspace(M, N, K):
    plan = dg.dg_describe_plan(dg.DG_OP_GEMM_NT, M, N, K)
    assert ("kernel=skinny" in plan) == ((M, N, K) in SKINNY + SKINNY_MID), plan
    a32, b32 = workloads.dense(M, N, K, seed=M + 3 * N + K)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    ws = _ws(M, N, K)
    outs = []
    for _ in range(3):
        D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
        dg.dg_fp8_gemm_nt(_t(qa), _t(sa), _t(qb), _t(sb), D, ws)
        outs.append(D)
    torch.cuda.synchronize()
    got = _np(outs[0]).view(np.uint16)
    for o in outs[1:]:
        assert np.array_equal(_np(o).view(np.uint16), got), "results differ between calls on one workspace"
    # a counter left non-zero by one call would leave tiles of the next call
    # unreduced (still -1), so equal results across calls show they were reset
    assert_close(got, oracle.gemm_nt(qa, sa, qb, sb), f"dense {M}x{N}x{K}")


# zero scales (an all-zero group quantised as amax / 448 gives alpha = 0, a
# zero weight block gives beta = 0): such blocks contribute exactly nothing,
# on the skinny (M <= 512 here) and the LDS-ring (M > 2048 here) paths,
# including a zero scale in the first and in the last K block of a row
@pytest.mark.parametrize("M,N,K", [(64, 272, 1024), (300, 272, 1024), (128, 2112, 7168), (512, 384, 640),
                                   (2100, 272, 1024), (2300, 384, 640)])
def test_dense_zero_scales_add_nothing(M, N, K):
    a32, b32 = workloads.dense(M, N, K, seed=M + N)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    rng = np.random.default_rng(M)
    KB = K // 128
    sa[rng.random(sa.shape) < 0.05] = 0.0
    sa[0, 1] = 0.0
    sa[KB - 1, 2] = 0.0
    sa[:, 3] = 0.0  # a row with every scale zero
    sb[0, KB - 1] = 0.0
    sb[-1, 0] = 0.0
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    for ws in (True, False):
        got = _gpu_dense(qa, sa, qb, sb, M, N, K, ws)
        assert not np.isnan(oracle.bf16_bits_to_f64(got)).any()
        assert_close(got, ref, f"dense {M}x{N}x{K} with zero scales")


# ---------------------------------------------------------------- contiguous

def _contig_small(counts, G, N, K, seed):
    w = workloads.contiguous(G, N, K, seed, counts=counts)
    qa, sa = oracle.quant_1x128(w["a"])
    qa, sa = workloads.place_rows(qa, sa, w["rows"], w["m_total"])
    qb, sb = oracle.quant_128x128(w["b"])
    return w, qa, sa, qb, sb


@pytest.mark.parametrize("counts,N,K", [([5, 130, 1], 144, 256), ([128, 256, 1, 300], 272, 512), ([1], 16, 128),
                                        ([129, 0, 7], 128, 384), ([700, 33, 256, 1], 400, 640)])
def test_contiguous_matches_oracle(counts, N, K):
    G = len(counts)
    w, qa, sa, qb, sb = _contig_small(counts, G, N, K, seed=sum(counts))
    D = _sentinel(w["m_total"], N)
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(w["m_indices"]))
    got = _np(D)
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, w["m_indices"], np.full((w["m_total"], N), SENTINEL, np.uint16))
    pad = w["m_indices"] < 0
    assert np.array_equal(got[pad], ref[pad])
    assert_close(got[~pad], ref[~pad], "contiguous")


def test_contiguous_out_of_range_indices_untouched():
    w, qa, sa, qb, sb = _contig_small([100, 60], 2, 128, 256, seed=3)
    idx = w["m_indices"].copy()
    idx[3] = 2  # == G
    idx[140] = -5
    idx[150] = 999
    D = _sentinel(w["m_total"], 128)
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(idx))
    got = _np(D)
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, idx, np.full((w["m_total"], 128), SENTINEL, np.uint16))
    bad = (idx < 0) | (idx >= 2)
    assert np.all(got[bad] == SENTINEL)
    assert_close(got[~bad], ref[~bad], "contiguous with out-of-range indices")


# ---------------------------------------------------------------- masked

@pytest.mark.parametrize("mm,max_m,N,K", [([64, 0, 17, 40], 64, 128, 256), ([256, 1, 129, 0, 200, 255], 256, 272, 512),
                                          ([3, 99, -4], 8, 16, 128), ([0, 0], 128, 128, 128),
                                          ([200, 128, 129, 73], 200, 528, 384),   # capacity not a multiple of 128
                                          ([300, 257, 1, 256], 300, 304, 256)])   # three 128-row tiles
def test_masked_matches_oracle(mm, max_m, N, K):
    G = len(mm)
    w = workloads.masked(G, max_m, N, K, seed=G + max_m, masked_m=mm)
    qa, sa = oracle.quant_1x128(w["a"]) if w["rows"].size else (np.zeros((0, K), np.uint8),
                                                                  np.zeros((K // 128, 0), np.float32))
    qa, sa = masked_layout(qa, sa, w["rows"], G, max_m)
    qb, sb = oracle.quant_128x128(w["b"])
    D = _sentinel(G, max_m, N)
    dg.dg_m_grouped_fp8_gemm_nt_masked(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(w["masked_m"]))
    got = _np(D)
    ref = oracle.grouped_masked(qa, sa, qb, sb, w["masked_m"], np.full((G, max_m, N), SENTINEL, np.uint16))
    valid = np.zeros((G, max_m), bool)
    for g, m in enumerate(w["masked_m"]):
        valid[g, :min(max(int(m), 0), max_m)] = True
    assert np.array_equal(got[~valid], ref[~valid])
    if valid.any():
        assert_close(got[valid], ref[valid], "masked")


def test_masked_graph_replay_with_device_side_counts():
    """Capture one masked call in a HIP graph, then change masked_m on the device
    between replays: each replay must follow the new counts with no re-capture."""
    G, max_m, N, K = 4, 128, 256, 512
    w = workloads.masked(G, max_m, N, K, seed=77, masked_m=[max_m] * G)
    qa, sa = oracle.quant_1x128(w["a"])
    qa, sa = masked_layout(qa, sa, w["rows"], G, max_m)
    qb, sb = oracle.quant_128x128(w["b"])
    A, SA, B, SB = _t(qa), _t(sa), _t(qb), _t(sb)
    mm_dev = torch.zeros(G, dtype=torch.int32, device=DEV)
    D = _sentinel(G, max_m, N)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside capture
        dg.dg_m_grouped_fp8_gemm_nt_masked(A, SA, B, SB, D, mm_dev)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.dg_m_grouped_fp8_gemm_nt_masked(A, SA, B, SB, D, mm_dev)
    for counts in ([128, 0, 5, 64], [1, 127, 0, 128], [0, 0, 0, 3]):
        D.fill_(-1)  # eager work between replays
        mm_dev.copy_(torch.tensor(counts, dtype=torch.int32))
        graph.replay()
        got = _np(D)
        ref = oracle.grouped_masked(qa, sa, qb, sb, np.array(counts), np.full((G, max_m, N), SENTINEL, np.uint16))
        valid = np.zeros((G, max_m), bool)
        for g, m in enumerate(counts):
            valid[g, :m] = True
        assert np.array_equal(got[~valid], ref[~valid]), counts
        assert_close(got[valid], ref[valid], f"graph replay {counts}")


# ---------------------------------------------------------------- few workgroups, many tiles each

@pytest.fixture
def few_cus():
    """Cap the persistent kernels at a few workgroups, so each walks many tiles
    (the LDS ring continues across tiles; a finished tile is stored while the
    next one computes; in the contiguous form the expert changes between
    tiles)."""
    def cap(n):
        dg.dg_set_num_cus(n)
    yield cap
    dg.dg_set_num_cus(0)


@pytest.mark.parametrize("cus", [1, 3, 7])
@pytest.mark.parametrize("M,N,K", [(1000, 528, 512), (777, 400, 384), (2048, 256, 1024)])
def test_dense_many_tiles_per_workgroup(few_cus, cus, M, N, K):
    few_cus(cus)
    a32, b32 = workloads.dense(M, N, K, seed=M + N + cus)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    for ws in (True, False):  # with a workspace the partial last round is split along K
        assert_close(_gpu_dense(qa, sa, qb, sb, M, N, K, ws), ref, f"dense {M}x{N}x{K} on {cus} CUs")


def _planned_kernel(capfd, fn):
    """Run fn with the planner's configuration printout on; return which dense kernel it chose."""
    os.environ["DG_PRINT_CONFIGS"] = "1"
    try:
        capfd.readouterr()
        fn()
        torch.cuda.synchronize()
        err = capfd.readouterr().err
    finally:
        del os.environ["DG_PRINT_CONFIGS"]
    return "wide" if "kernel=wide" in err else ("persistent" if "kernel=persistent" in err else "other")


# (cus, M, N, K, kernel): 256 x 256 tiles are planned when they fill whole
# rounds of the CUs to >= 85% or make one round on >= 60% of them, else
# 256 x 128 tiles with a K-split tail
WIDE_CASES = [(1, 256, 256, 128, "wide"), (4, 512, 512, 640, "wide"), (4, 500, 496, 384, "wide"),
              (3, 300, 608, 1024, "wide"), (7, 1000, 1792, 512, "wide"), (2, 1024, 272, 256, "wide"),
              (10, 768, 512, 512, "wide"), (10, 1280, 256, 512, "persistent"),
              (7, 2048, 256, 1024, "persistent"), (5, 777, 400, 384, "persistent")]


@pytest.mark.parametrize("cus,M,N,K,kernel", WIDE_CASES)
def test_dense_wide_and_persistent_planning(few_cus, capfd, cus, M, N, K, kernel):
    few_cus(cus)
    a32, b32 = workloads.dense(M, N, K, seed=M + 2 * N + cus)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    out = {}
    assert _planned_kernel(capfd, lambda: out.setdefault("d", _gpu_dense(qa, sa, qb, sb, M, N, K))) == kernel
    assert_close(out["d"], oracle.gemm_nt(qa, sa, qb, sb), f"dense {M}x{N}x{K} on {cus} CUs ({kernel})")


def test_dense_wide_deterministic_and_untouched_outside():
    # the wide kernel writes exactly the M x N output (D sits inside a larger
    # sentinel buffer) and repeats bit for bit
    M, N, K = 500, 496, 384
    dg.dg_set_num_cus(4)
    try:
        a32, b32 = workloads.dense(M, N, K, seed=5)
        qa, sa = oracle.quant_1x128(a32)
        qb, sb = oracle.quant_128x128(b32)
        big = torch.full((M + 8, N), -1, dtype=torch.int16, device=DEV)
        D = big[4:4 + M]
        dg.dg_fp8_gemm_nt(_t(qa), _t(sa), _t(qb), _t(sb), D)
        first = _np(D).copy()
        dg.dg_fp8_gemm_nt(_t(qa), _t(sa), _t(qb), _t(sb), D)
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(0)
    assert np.array_equal(first, _np(D))
    rest = big.cpu().numpy()
    assert (rest[:4] == -1).all() and (rest[4 + M:] == -1).all()
    assert_close(first, oracle.gemm_nt(qa, sa, qb, sb), "wide 500x496x384")


@pytest.mark.parametrize("cus", [1, 4])
@pytest.mark.parametrize("counts,N,K", [([130, 5, 300, 1, 256], 400, 384), ([128, 0, 900, 77], 528, 256)])
def test_contiguous_many_tiles_per_workgroup(few_cus, cus, counts, N, K):
    few_cus(cus)
    G = len(counts)
    w, qa, sa, qb, sb = _contig_small(counts, G, N, K, seed=sum(counts) + cus)
    idx = w["m_indices"].copy()
    idx[1] = G + 3  # out of range: untouched
    D = _sentinel(w["m_total"], N)
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(idx))
    got = _np(D)
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, idx, np.full((w["m_total"], N), SENTINEL, np.uint16))
    bad = (idx < 0) | (idx >= G)
    assert np.array_equal(got[bad], ref[bad])
    assert np.all(got[bad] == SENTINEL)
    assert_close(got[~bad], ref[~bad], f"contiguous on {cus} CUs")


# (cus, counts, N, K, kernel): 256 x 256 tiles (two half passes where a tile
# straddles two experts) when they fill whole rounds to >= 85%, at any K
CONTIG_WIDE = [(1, [130, 5, 300, 1, 256], 400, 4096, "wide"), (2, [256, 256, 100], 272, 4224, "wide"),
               (4, [300, 256, 256], 528, 4096, "wide"), (3, [130, 5, 300, 1, 256], 400, 4096, "persistent"),
               (1, [130, 5, 300, 1, 256], 400, 2048, "wide"), (3, [130, 5, 300, 1, 256], 400, 1024, "persistent")]


@pytest.mark.parametrize("cus,counts,N,K,kernel", CONTIG_WIDE)
def test_contiguous_wide_planning_and_passes(few_cus, capfd, cus, counts, N, K, kernel):
    few_cus(cus)
    G = len(counts)
    w, qa, sa, qb, sb = _contig_small(counts, G, N, K, seed=sum(counts) + 7 * cus)
    idx = w["m_indices"].copy()
    if len(counts) == 3 and counts[0] == 300:
        idx[:256] = -1          # a whole 256-row tile without a valid index: no pass
        idx[300] = G + 1        # out of range inside a padded block: untouched
    D = _sentinel(w["m_total"], N)
    got_kernel = _planned_kernel(capfd, lambda: dg.dg_m_grouped_fp8_gemm_nt_contiguous(
        _t(qa), _t(sa), _t(qb), _t(sb), D, _t(idx)))
    assert got_kernel == kernel
    got = _np(D)
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, idx, np.full((w["m_total"], N), SENTINEL, np.uint16))
    bad = (idx < 0) | (idx >= G)
    assert np.all(got[bad] == SENTINEL)
    assert_close(got[~bad], ref[~bad], f"contiguous {counts} on {cus} CUs ({kernel})")


@pytest.mark.parametrize("cus", [1, 5])
def test_masked_many_tiles_per_workgroup(few_cus, cus):
    few_cus(cus)
    mm, max_m, N, K = [256, 3, 0, 200, 129, 256], 256, 400, 384
    G = len(mm)
    w = workloads.masked(G, max_m, N, K, seed=cus + 11, masked_m=mm)
    qa, sa = oracle.quant_1x128(w["a"])
    qa, sa = masked_layout(qa, sa, w["rows"], G, max_m)
    qb, sb = oracle.quant_128x128(w["b"])
    D = _sentinel(G, max_m, N)
    dg.dg_m_grouped_fp8_gemm_nt_masked(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(w["masked_m"]))
    got = _np(D)
    ref = oracle.grouped_masked(qa, sa, qb, sb, w["masked_m"], np.full((G, max_m, N), SENTINEL, np.uint16))
    valid = np.zeros((G, max_m), bool)
    for g, m in enumerate(mm):
        valid[g, :m] = True
    assert np.array_equal(got[~valid], ref[~valid])
    assert_close(got[valid], ref[valid], f"masked on {cus} CUs")
