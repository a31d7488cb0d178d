"""Accumulating FP8 GEMM (dg_fp8_gemm_nt_acc, D = C + A.B^T in fp32) against
the oracle (oracle.gemm_nt_c): skinny (M <= 128, and up to 2048 rows with
few columns or short K), persistent (other M > 128) and wide (256 x 256
tiles) kernels, with C given, absent and aliased to D, with
and without K splits, many tiles per workgroup; integer inputs bit-exact; the
4096 x 7168 x 16384 shape in place at full size on sampled rows and columns."""

import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import acc_tolerance, assert_f32_rule

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _ws(M, N, K):
    n = dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT, M, N, K, 1)
    return torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV) if n else None


def _case(M, N, K, seed):
    a32, b32 = workloads.dense(M, N, K, seed)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    rng = np.random.default_rng(seed + 1)
    c = (rng.standard_normal((M, N)) * 3.0).astype(np.float32)
    return qa, sa, qb, sb, c


def _check(got, qa, sa, qb, sb, c, what):
    ref = oracle.gemm_nt_c(qa, sa, qb, sb, c)
    tol = acc_tolerance(qa, sa, qb, sb, c)
    bad = ~(np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= tol)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the bound, e.g. " \
                          f"{[(tuple(i), float(got[tuple(i)]), float(ref[tuple(i)])) for i in np.argwhere(bad)[:3]]}"
    # the per-element acceptance rule on top of the arithmetic ceiling above
    assert_f32_rule(got, ref, what)


SHAPES = [(1, 16, 128), (64, 2112, 1024), (100, 272, 4096), (128, 528, 512), (130, 144, 640), (250, 1008, 3072),
          (257, 400, 384), (400, 2112, 1024), (333, 1536, 7168), (257, 7168, 1024), (200, 144, 9216),
          (700, 1536, 1024), (777, 2112, 1024), (2100, 400, 384), (1000, 528, 512), (2048, 256, 1024)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("mode", ["c", "none", "inplace"])
@pytest.mark.parametrize("workspace", [True, False])
def test_acc_matches_oracle(M, N, K, mode, workspace):
    qa, sa, qb, sb, c = _case(M, N, K, seed=M + N + K)
    C = None if mode == "none" else _t(c)
    D = C if mode == "inplace" else torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), C, D, _ws(M, N, K) if workspace else None)
    torch.cuda.synchronize()
    _check(D.cpu().numpy(), qa, sa, qb, sb, None if mode == "none" else c, f"acc {M}x{N}x{K} {mode}")


@pytest.mark.parametrize("cus", [1, 5])
@pytest.mark.parametrize("M,N,K", [(777, 400, 384), (64, 2112, 1024)])
def test_acc_many_tiles_per_workgroup(cus, M, N, K):
    dg.dg_set_num_cus(cus)
    try:
        qa, sa, qb, sb, c = _case(M, N, K, seed=cus * 7 + M)
        ws = _ws(M, N, K)
        D = torch.empty((M, N), dtype=torch.float32, device=DEV)
        dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), _t(c), D, ws)
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(0)
    _check(D.cpu().numpy(), qa, sa, qb, sb, c, f"acc {M}x{N}x{K} on {cus} CUs")


# (cus, M, N, K): 256 x 256 tiles (the wide kernel, C loaded and D stored
# row tile by row tile) once they fill whole rounds of the capped CUs
WIDE = [(1, 256, 256, 128), (4, 512, 512, 640), (4, 500, 496, 384), (3, 300, 608, 1024), (7, 1000, 1792, 512)]


@pytest.mark.parametrize("cus,M,N,K", WIDE)
@pytest.mark.parametrize("mode", ["c", "none", "inplace"])
def test_acc_wide_tiles(capfd, cus, M, N, K, mode):
    dg.dg_set_num_cus(cus)
    os.environ["DG_PRINT_CONFIGS"] = "1"
    try:
        qa, sa, qb, sb, c = _case(M, N, K, seed=cus + M + N)
        C = None if mode == "none" else _t(c)
        D = C if mode == "inplace" else torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        capfd.readouterr()
        dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), C, D, _ws(M, N, K))
        torch.cuda.synchronize()
        assert "kernel=wide" in capfd.readouterr().err
    finally:
        del os.environ["DG_PRINT_CONFIGS"]
        dg.dg_set_num_cus(0)
    _check(D.cpu().numpy(), qa, sa, qb, sb, None if mode == "none" else c, f"acc wide {M}x{N}x{K} {mode} on {cus} CUs")


def test_acc_wide_integer_inputs_bit_exact():
    M, N, K = 512, 496, 512
    dg.dg_set_num_cus(4)
    try:
        rng = np.random.default_rng(9)
        qa = oracle.encode_e4m3(rng.integers(-10, 10, (M, K)).astype(np.float32))
        qb = oracle.encode_e4m3(rng.integers(-10, 10, (N, K)).astype(np.float32))
        sa = np.ones((K // 128, M), np.float32)
        sb = np.ones(((N + 127) // 128, K // 128), np.float32)
        c = rng.integers(-5000, 5000, (M, N)).astype(np.float32)
        D = _t(c)  # in place
        dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), D, D, None)
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(0)
    assert np.array_equal(D.cpu().numpy(), oracle.gemm_nt_c(qa, sa, qb, sb, c))


@pytest.mark.parametrize("M,N,K", [(64, 272, 512), (300, 144, 1024)])
def test_acc_integer_inputs_bit_exact(M, N, K):
    # integers in [-10, 9] with unit scales and integer C: every partial, sum and
    # C + sum is an integer below 2^24, so the fp32 result equals the oracle's
    rng = np.random.default_rng(M)
    qa = oracle.encode_e4m3(rng.integers(-10, 10, (M, K)).astype(np.float32))
    qb = oracle.encode_e4m3(rng.integers(-10, 10, (N, K)).astype(np.float32))
    sa = np.ones((K // 128, M), np.float32)
    sb = np.ones(((N + 127) // 128, K // 128), np.float32)
    c = rng.integers(-5000, 5000, (M, N)).astype(np.float32)
    ref = oracle.gemm_nt_c(qa, sa, qb, sb, c)
    for ws in (True, False):
        D = torch.empty((M, N), dtype=torch.float32, device=DEV)
        dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), _t(c), D, _ws(M, N, K) if ws else None)
        torch.cuda.synchronize()
        assert np.array_equal(D.cpu().numpy(), ref)


@pytest.mark.timeout(600)
def test_acc_full_size_in_place():
    # the accumulate workload's shape and configuration: C = D in place, 256 x 256 tiles
    M, N, K, seed = 4096, 7168, 16384, 200
    a32, b32 = workloads.dense(M, N, K, seed)
    A32, B32 = _t(a32), _t(b32)
    A = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    SA = torch.empty((K // 128, M), dtype=torch.float32, device=DEV)
    B = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    SB = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=DEV)
    dg.dg_quant_1x128(A32, A, SA)
    dg.dg_quant_128x128(B32, B, SB)
    del A32, B32
    rng = np.random.default_rng(seed + 1)
    c = (rng.standard_normal((M, N)) * 3.0).astype(np.float32)
    D = _t(c)
    dg.dg_fp8_gemm_nt_acc(A, SA, B, SB, D, D, _ws(M, N, K))
    torch.cuda.synchronize()
    rows = np.array(sorted({0, M // 2, M - 1} | set(int(r) for r in rng.integers(0, M, 9))))
    ri = torch.from_numpy(rows).to(DEV)
    qa, sa = oracle.quant_1x128(a32[rows])
    assert np.array_equal(A.index_select(0, ri).cpu().numpy(), qa)
    got = D.index_select(0, ri).cpu().numpy()
    for blk in (0, 27, 55):
        c0, c1 = 128 * blk, 128 * blk + 128
        qb, sb = oracle.quant_128x128(b32[c0:c1])
        _check(got[:, c0:c1], qa, sa, qb, sb, c[rows][:, c0:c1], f"acc full size columns {c0}:{c1}")


def test_mfma_dot_product_truncation_bound():
    # one K block, unit scales: a row of 448 followed by 127 copies of 2^-j and
    # a row of ones in B.  The exact sum is 448 + 127 * 2^-j; the matrix cores
    # may drop or truncate the small terms that share an 8-term group with 448,
    # but never by more than 2^-10 * sum |a*b| (the bound acc_tolerance uses)
    K, N = 128, 16
    js = list(range(-9, 10))
    A = np.zeros((len(js), K), np.float32)
    for i, j in enumerate(js):
        A[i, 0] = 448.0
        A[i, 1:] = 2.0 ** (-j)
    qa = oracle.encode_e4m3(A)
    qb = oracle.encode_e4m3(np.ones((N, K), np.float32))
    sa = np.ones((1, len(js)), np.float32)
    sb = np.ones((1, 1), np.float32)
    D = torch.empty((len(js), N), dtype=torch.float32, device=DEV)
    dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), None, D)
    torch.cuda.synchronize()
    got = D.cpu().numpy().astype(np.float64)
    exact = oracle.decode_e4m3(qa).sum(axis=1)[:, None]
    assert np.all(np.abs(got - exact) <= 2.0 ** -10 * np.abs(exact))
    _check(D.cpu().numpy(), qa, sa, qb, sb, None, "truncation probe")
