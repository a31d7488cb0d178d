"""BF16 dense GEMM (dg_bf16_gemm_nt) against the oracle (oracle/gemm_bf16.py):
small and ragged shapes on one or many tiles per workgroup, with and without
a K-split tail and on 256 x 256 tiles, integer inputs bit-exact, and the full
4096 x 7168 x 16384 shape on sampled rows."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16) if x.dtype == np.uint16 else x).to(DEV)


def _run(a, b, workspace=True, reuse=None):
    M, K = a.shape
    N = b.shape[0]
    ws = reuse
    if ws is None and workspace:
        n = dg.dg_get_workspace_size(dg.DG_OP_BF16_GEMM_NT, M, N, K, 1)
        ws = torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV) if n else None
    D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
    dg.dg_bf16_gemm_nt(_t(a), _t(b), D, ws)
    torch.cuda.synchronize()
    return D.cpu().numpy().view(np.uint16)


SHAPES = [(1, 16, 64), (64, 2112, 512), (130, 144, 640), (257, 400, 384), (777, 2112, 640), (1000, 528, 512),
          (2048, 256, 1024), (300, 272, 64), (256, 128, 192)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("workspace", [True, False])
def test_bf16_matches_oracle(M, N, K, workspace):
    a, b = workloads.dense_bf16(M, N, K, seed=M + 2 * N + K)
    assert_close(_run(a, b, workspace), oracle.gemm_bf16_nt(a, b), f"bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 272, 512), (200, 144, 1024), (513, 400, 128)])
def test_bf16_integer_inputs_bit_exact(M, N, K):
    # integers in [-3, 3]: products and fp32 sums are exact (|sum| <= 9 K < 2^24),
    # and the results, integers below 2^8 or rounded once, must equal the oracle's bits
    rng = np.random.default_rng(M)
    a = oracle.bf16_rne_bits(rng.integers(-3, 4, (M, K)).astype(np.float64))
    b = oracle.bf16_rne_bits(rng.integers(-3, 4, (N, K)).astype(np.float64))
    ref = oracle.gemm_bf16_nt(a, b)
    for ws in (True, False):
        assert np.array_equal(_run(a, b, ws), ref)


@pytest.mark.parametrize("cus", [1, 3, 7])
@pytest.mark.parametrize("M,N,K", [(1000, 528, 512), (777, 400, 384)])
def test_bf16_many_tiles_per_workgroup_reused_workspace(cus, M, N, K):
    dg.dg_set_num_cus(cus)
    try:
        a, b = workloads.dense_bf16(M, N, K, seed=cus + M)
        n = dg.dg_get_workspace_size(dg.DG_OP_BF16_GEMM_NT, M, N, K, 1)
        ws = torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV)
        outs = [_run(a, b, reuse=ws) for _ in range(3)]
    finally:
        dg.dg_set_num_cus(0)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), "results differ between calls on one workspace"
    assert_close(outs[0], oracle.gemm_bf16_nt(a, b), f"bf16 {M}x{N}x{K} on {cus} CUs")


# (cus, M, N, K): 256 x 256 tiles (the wide kernel) once they fill whole rounds
# of the (capped) CUs: ragged M and N, several tiles per workgroup, one K block
WIDE = [(1, 256, 256, 64), (4, 512, 512, 640), (4, 500, 496, 384), (3, 300, 608, 1024), (2, 1024, 272, 256),
        (7, 1000, 1792, 512)]


@pytest.mark.parametrize("cus,M,N,K", WIDE)
def test_bf16_wide_tiles(cus, M, N, K):
    dg.dg_set_num_cus(cus)
    try:
        assert "kernel=wide" in dg.dg_describe_plan(dg.DG_OP_BF16_GEMM_NT, M, N, K, 1)
        a, b = workloads.dense_bf16(M, N, K, seed=cus + M + N)
        got = _run(a, b)
        rng = np.random.default_rng(M + N)  # integers in [-3, 3]: exact products and sums
        ai = oracle.bf16_rne_bits(rng.integers(-3, 4, (M, K)).astype(np.float64))
        bi = oracle.bf16_rne_bits(rng.integers(-3, 4, (N, K)).astype(np.float64))
        got_i = _run(ai, bi)
    finally:
        dg.dg_set_num_cus(0)
    assert_close(got, oracle.gemm_bf16_nt(a, b), f"bf16 wide {M}x{N}x{K} on {cus} CUs")
    assert np.array_equal(got_i, oracle.gemm_bf16_nt(ai, bi))


def test_bf16_full_size_sampled_rows():
    M, N, K = 4096, 7168, 16384
    a, b = workloads.dense_bf16(M, N, K, seed=500)
    got = _run(a, b)
    assert not np.isnan(oracle.bf16_bits_to_f64(got)).any()
    rows = np.array([0, 1, 255, 256, 2047, 4000, 4095])
    assert_close(got[rows], oracle.gemm_bf16_nt(a[rows], b), "bf16 full size, sampled rows")


def test_bf16_shape_errors():
    a = torch.zeros((64, 96), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((16, 96), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros((64, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dg.DGError):
        dg.dg_bf16_gemm_nt(a, b, d)  # K = 96 is not a multiple of 64
