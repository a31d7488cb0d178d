"""UE8M0 (power-of-two) scale variant on the GPU against the oracle
(oracle/ue8m0.py): both quantisers bit-exact (bytes and packed code words,
ragged N, K blocks not a multiple of four, several groups, zero groups,
amax exactly at and just past the power-of-two boundaries, tiny values), the
GEMM within the bf16 tolerance over small, ragged and split shapes, on
256 x 256 tiles and on the skinny (rows <= 2048) kernel's every compiled
configuration, bit identity with the fp32-scale kernels fed the same powers
of two, and the
4096x7168x16384 shape at full size on sampled rows and column blocks."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from oracle.ue8m0 import ue8m0_value, unpack_k
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _kw(K):
    return (K // 128 + 3) // 4


def _edge_rows(M, K, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-30, 30, (M, 1)))).astype(np.float32)
    if M >= 8 and K >= 256:
        x[0, :128] = 0.0                                   # all-zero group
        x[1, 5] = np.float32(448.0)                        # amax exactly 448 * 2^0
        x[1, :128] = np.clip(x[1, :128], -400, 400)
        x[1, 5] = np.float32(448.0)
        x[2, 7] = np.nextafter(np.float32(448.0 * 8), np.float32(np.inf))  # just past a boundary
        x[3, 128:256] *= np.float32(1e-38)                 # tiny (subnormal amax)
        x[4, 130] = np.float32(-3.0e38)                    # huge
    return x


# the last case has 65688 groups: a grid of over 4096 workgroups whose last
# one is partly filled
@pytest.mark.parametrize("G,M,K", [(1, 64, 128), (1, 37, 640), (3, 20, 1024), (1, 300, 512), (2, 9, 1152),
                                   (3, 391, 7168)])
def test_quant_1x128_ue8m0_bit_exact(G, M, K):
    x = np.stack([_edge_rows(M, K, 10 * g + K) for g in range(G)])
    q = torch.empty((G, M, K), dtype=torch.uint8, device=DEV)
    s = torch.full((G, _kw(K), M), -1, dtype=torch.int32, device=DEV)  # unused bytes must be cleared
    dg.dg_quant_1x128_ue8m0(_t(x), q, s)
    torch.cuda.synchronize()
    for g in range(G):
        rq, _, rs = oracle.quant_1x128_ue8m0(x[g])
        assert np.array_equal(q[g].cpu().numpy(), rq), f"bytes of group {g}"
        assert np.array_equal(s[g].cpu().numpy(), rs), f"packed codes of group {g}"


@pytest.mark.parametrize("G,N,K", [(1, 128, 128), (1, 200, 640), (2, 384, 512), (1, 16, 1152)])
def test_quant_128x128_ue8m0_bit_exact(G, N, K):
    x = np.stack([_edge_rows(N, K, 20 * g + N) for g in range(G)])
    q = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    s = torch.full((G, (N + 127) // 128, _kw(K)), -1, dtype=torch.int32, device=DEV)
    dg.dg_quant_128x128_ue8m0(_t(x), q, s)
    torch.cuda.synchronize()
    for g in range(G):
        rq, _, rs = oracle.quant_128x128_ue8m0(x[g])
        assert np.array_equal(q[g].cpu().numpy(), rq), f"bytes of group {g}"
        assert np.array_equal(s[g].cpu().numpy(), rs), f"packed codes of group {g}"


def _case(M, N, K, seed):
    a32, b32 = workloads.dense(M, N, K, seed)
    qa, _, pa = oracle.quant_1x128_ue8m0(a32)
    qb, _, pb = oracle.quant_128x128_ue8m0(b32)
    return qa, pa, qb, pb


def _ws(M, N, K):
    n = dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT_UE8M0, M, N, K, 1)
    return torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV) if n else None


SHAPES = [(1, 16, 128), (64, 2112, 1024), (128, 272, 640), (257, 400, 384), (2100, 400, 384), (1000, 528, 512),
          (2048, 256, 1152),
          (4096, 256, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("workspace", [True, False])
def test_gemm_ue8m0_matches_oracle(M, N, K, workspace):
    qa, pa, qb, pb = _case(M, N, K, seed=M + 3 * N + K)
    D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.dg_fp8_gemm_nt_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D, _ws(M, N, K) if workspace else None)
    torch.cuda.synchronize()
    ref = oracle.gemm_nt_ue8m0(qa, pa, qb, pb)
    assert_close(D.view(torch.int16).cpu().numpy().view(np.uint16), ref, f"ue8m0 {M}x{N}x{K}")


@pytest.mark.parametrize("cus", [1, 6])
def test_gemm_ue8m0_many_tiles_per_workgroup(cus):
    M, N, K = 777, 400, 384
    dg.dg_set_num_cus(cus)
    try:
        qa, pa, qb, pb = _case(M, N, K, seed=cus)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        dg.dg_fp8_gemm_nt_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D, _ws(M, N, K))
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(0)
    assert_close(D.view(torch.int16).cpu().numpy().view(np.uint16), oracle.gemm_nt_ue8m0(qa, pa, qb, pb),
                 f"ue8m0 on {cus} CUs")


# (cus, M, N, K): 256 x 256 tiles (the wide kernel) once they fill whole rounds
# of the (capped) CUs, ragged M and N included, several tiles per workgroup
WIDE = [(1, 256, 256, 128), (4, 512, 512, 640), (4, 500, 496, 384), (3, 300, 608, 1024), (2, 1024, 272, 256)]


@pytest.mark.parametrize("cus,M,N,K", WIDE)
def test_gemm_ue8m0_wide_tiles(cus, M, N, K):
    dg.dg_set_num_cus(cus)
    try:
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT_UE8M0, M, N, K, 1)
        qa, pa, qb, pb = _case(M, N, K, seed=cus + M + N)
        D = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        dg.dg_fp8_gemm_nt_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D, _ws(M, N, K))
        # the fp32-scale kernel on the same plan, fed the same powers of two: bit for bit
        kb = K // 128
        D2 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        dg.dg_fp8_gemm_nt(_t(qa), _t(ue8m0_value(unpack_k(pa.T, kb).T)), _t(qb), _t(ue8m0_value(unpack_k(pb, kb))), D2)
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(0)
    assert torch.equal(D.view(torch.int16), D2.view(torch.int16))
    assert_close(D.view(torch.int16).cpu().numpy().view(np.uint16), oracle.gemm_nt_ue8m0(qa, pa, qb, pb),
                 f"ue8m0 wide {M}x{N}x{K} on {cus} CUs")


@pytest.mark.parametrize("M,N,K", [(300, 400, 640), (2048, 1024, 2048)])
def test_gemm_ue8m0_bit_identical_to_fp32_scale_kernel(M, N, K):
    # the same powers of two as fp32 scales: the matrix cores' exact scaling
    # followed by one add equals the fp32 path's multiply-add, bit for bit
    qa, pa, qb, pb = _case(M, N, K, seed=7 + M)
    kb = K // 128
    sa = ue8m0_value(unpack_k(pa.T, kb).T)
    sb = ue8m0_value(unpack_k(pb, kb))
    D1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    D2 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dg.dg_fp8_gemm_nt_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D1, _ws(M, N, K))
    dg.dg_fp8_gemm_nt(_t(qa), _t(sa), _t(qb), _t(sb), D2, _ws(M, N, K))
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))


# (M, N, K, forced plan): rows <= 128 (and up to 2048 rows with few columns) run
# the skinny kernel; the forced plans reach every compiled (tile rows, columns
# per wave, ring depth) instance with a K split, ragged M and N, and K blocks
# not a multiple of four, also with several row tiles
SKINNY = [(1, 16, 128, None), (37, 400, 640, None), (100, 528, 1152, None), (64, 2112, 7168, None),
          (128, 7168, 2048, None), (160, 2112, 7168, None), (230, 528, 1152, None),
          (50, 272, 640, "skinny=64x16x2x4"), (64, 400, 1024, "skinny=64x16x3x8"),
          (64, 528, 1152, "skinny=64x32x3x4"), (61, 528, 1024, "skinny=64x32x2x6"),
          (128, 272, 896, "skinny=128x16x2x6"), (120, 528, 1152, "skinny=128x32x3x4"),
          (200, 528, 1152, "skinny=64x32x3x4"), (256, 272, 896, "skinny=128x16x2x6"),
          (170, 528, 1152, "skinny=128x32x3x4"), (400, 2112, 1024, None), (257, 7168, 1024, None),
          (333, 1536, 3072, None), (450, 528, 1152, "skinny=64x16x3x8"), (500, 400, 1024, "skinny=128x16x2x6"),
          (520, 1008, 7168, None), (700, 1536, 5120, None), (1500, 272, 896, "skinny=128x32x2x4")]


@pytest.mark.parametrize("M,N,K,force", SKINNY)
def test_gemm_ue8m0_skinny(M, N, K, force, monkeypatch):
    if force:
        monkeypatch.setenv("DG_FORCE_CONFIG", force)
    plan = dg.dg_describe_plan(dg.DG_OP_GEMM_NT_UE8M0, M, N, K, 1)
    assert "kernel=skinny" in plan
    if force:
        assert f"splits={force.split('x')[2]}" in plan
    qa, pa, qb, pb = _case(M, N, K, seed=11 * M + N + K)
    kb = K // 128
    ws = torch.zeros(16 << 20, dtype=torch.float32, device=DEV)  # the same plan for both forms
    D1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    D2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dg.dg_fp8_gemm_nt_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D1, ws)
    # the fp32-scale skinny kernel fed the same powers of two: bit for bit
    dg.dg_fp8_gemm_nt(_t(qa), _t(ue8m0_value(unpack_k(pa.T, kb).T)), _t(qb), _t(ue8m0_value(unpack_k(pb, kb))), D2, ws)
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))
    assert_close(D1.view(torch.int16).cpu().numpy().view(np.uint16), oracle.gemm_nt_ue8m0(qa, pa, qb, pb),
                 f"ue8m0 skinny {M}x{N}x{K} {force or 'default plan'}")


@pytest.mark.timeout(600)
def test_gemm_ue8m0_full_size():
    M, N, K, seed = 4096, 7168, 16384, 200
    a32, b32 = workloads.dense(M, N, K, seed)
    A32, B32 = _t(a32), _t(b32)
    A = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    SA = torch.empty((_kw(K), M), dtype=torch.int32, device=DEV)
    B = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    SB = torch.empty(((N + 127) // 128, _kw(K)), dtype=torch.int32, device=DEV)
    dg.dg_quant_1x128_ue8m0(A32, A, SA)
    dg.dg_quant_128x128_ue8m0(B32, B, SB)
    del A32, B32
    D = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dg.dg_fp8_gemm_nt_ue8m0(A, SA, B, SB, D, _ws(M, N, K))
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = np.array(sorted({0, M // 2, M - 1} | set(int(r) for r in rng.integers(0, M, 9))))
    qa, _, pa = oracle.quant_1x128_ue8m0(a32[rows])
    ri = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(A[ri].cpu().numpy(), qa)
    assert np.array_equal(SA[:, ri].cpu().numpy(), pa)
    got = D.view(torch.int16).cpu().numpy().view(np.uint16)
    for blk in (0, 27, 55):
        c0, c1 = 128 * blk, 128 * blk + 128
        qb, _, pb = oracle.quant_128x128_ue8m0(b32[c0:c1])
        assert np.array_equal(B[c0:c1].cpu().numpy(), qb)
        assert np.array_equal(SB[blk:blk + 1].cpu().numpy(), pb)
        assert_close(got[rows, c0:c1], oracle.gemm_nt_ue8m0(qa, pa, qb, pb), f"full size columns {c0}:{c1}")
