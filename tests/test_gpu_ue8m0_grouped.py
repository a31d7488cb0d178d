"""M-grouped contiguous and masked GEMMs with UE8M0 scales
(dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0 / _masked_ue8m0) against the
oracle's compositions (oracle.grouped_contiguous_ue8m0 / grouped_masked_ue8m0,
pinned per expert to exact rational arithmetic): activations and weights
quantised by the library's own UE8M0 quantisers (checked bit-exact against the
oracle's), ragged expert sizes, padding rows and rows past masked_m left
bit-exact untouched, both tile kernels of the contiguous form, many tiles per
workgroup, bit identity with the fp32-scale grouped kernels fed the same
powers of two, the masked form replayed from a captured graph with masks
changed on the device, and the 32-expert decode configuration at full size on
sampled experts."""

import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from oracle.ue8m0 import ue8m0_value, unpack_k
from tests.helpers import SENTINEL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _kw(K):
    return (K // 128 + 3) // 4


def _quant_act(x):
    """Library UE8M0 activation quantiser on x [G, M, K] (or [M, K]); checked
    bit-exact against the oracle's."""
    X = _t(x)
    q = torch.empty(X.shape, dtype=torch.uint8, device=DEV)
    s = torch.empty(X.shape[:-2] + (_kw(x.shape[-1]), x.shape[-2]), dtype=torch.int32, device=DEV)
    dg.dg_quant_1x128_ue8m0(X, q, s)
    torch.cuda.synchronize()
    flat = x.reshape(-1, x.shape[-2], x.shape[-1])
    for g in range(flat.shape[0]):
        rq, _, rs = oracle.quant_1x128_ue8m0(flat[g])
        assert np.array_equal(q.reshape(flat.shape).cpu().numpy()[g], rq)
        assert np.array_equal(s.reshape((flat.shape[0],) + s.shape[-2:]).cpu().numpy()[g], rs)
    return q, s


def _quant_w(b):
    B = _t(b)
    G, N, K = b.shape
    q = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    s = torch.empty((G, (N + 127) // 128, _kw(K)), dtype=torch.int32, device=DEV)
    dg.dg_quant_128x128_ue8m0(B, q, s)
    torch.cuda.synchronize()
    for g in range(G):
        rq, _, rs = oracle.quant_128x128_ue8m0(b[g])
        assert np.array_equal(q[g].cpu().numpy(), rq) and np.array_equal(s[g].cpu().numpy(), rs)
    return q, s


def _contig(counts, N, K, seed):
    G = len(counts)
    w = workloads.contiguous(G, N, K, seed, counts=counts)
    # quantise the valid rows, then place them (padding rows: e4m3 NaN codes, zero scale words)
    qv, sv = _quant_act(w["a"])
    m_total = w["m_total"]
    A = torch.full((m_total, K), workloads.TRAP_CODE, dtype=torch.uint8, device=DEV)
    SA = torch.zeros((_kw(K), m_total), dtype=torch.int32, device=DEV)
    rows = torch.from_numpy(w["rows"]).to(DEV)
    A[rows] = qv
    SA[:, rows] = sv
    B, SB = _quant_w(w["b"])
    return w, A, SA, B, SB


CONTIG = [(0, [5, 130, 1], 144, 256, "persistent"), (0, [128, 256, 1, 300], 272, 512, "persistent"),
          (1, [130, 5, 300, 1, 256], 400, 4096, "wide"), (2, [256, 256, 100], 272, 4224, "wide"),
          (3, [700, 33, 256, 1], 400, 640, "persistent")]


@pytest.mark.parametrize("cus,counts,N,K,kernel", CONTIG)
def test_contiguous_ue8m0_matches_oracle(capfd, cus, counts, N, K, kernel):
    w, A, SA, B, SB = _contig(counts, N, K, seed=sum(counts) + K)
    D = torch.full((w["m_total"], N), -1, dtype=torch.int16, device=DEV)
    os.environ["DG_PRINT_CONFIGS"] = "1"
    dg.dg_set_num_cus(cus)
    try:
        capfd.readouterr()
        dg.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(A, SA, B, SB, D, _t(w["m_indices"]))
        torch.cuda.synchronize()
        assert f"kernel={kernel}" in capfd.readouterr().err
    finally:
        del os.environ["DG_PRINT_CONFIGS"]
        dg.dg_set_num_cus(0)
    got = _bits(D)
    ref = oracle.grouped_contiguous_ue8m0(A.cpu().numpy(), SA.cpu().numpy(), B.cpu().numpy(), SB.cpu().numpy(),
                                          w["m_indices"], np.full(got.shape, SENTINEL, np.uint16))
    pad = w["m_indices"] < 0
    assert np.array_equal(got[pad], ref[pad])
    assert_close(got[~pad], ref[~pad], f"contiguous ue8m0 {counts} on {kernel}")


def _decode_act(sp, kb):
    return ue8m0_value(np.swapaxes(unpack_k(np.swapaxes(sp, -1, -2), kb), -1, -2))


@pytest.mark.parametrize("cus,K", [(0, 512), (1, 4096)])  # 128 x 256 tiles; 256 x 256 tiles
def test_contiguous_ue8m0_bit_identical_to_fp32_scale_kernel(cus, K):
    counts, N = [130, 5, 300, 1, 256], 400
    w, A, SA, B, SB = _contig(counts, N, K, seed=K)
    kb = K // 128
    sa = _t(_decode_act(SA.cpu().numpy(), kb))
    sb = _t(ue8m0_value(unpack_k(SB.cpu().numpy(), kb)))
    idx = _t(w["m_indices"])
    D1 = torch.full((w["m_total"], N), -1, dtype=torch.int16, device=DEV)
    D2 = torch.full((w["m_total"], N), -1, dtype=torch.int16, device=DEV)
    dg.dg_set_num_cus(cus)
    try:
        dg.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(A, SA, B, SB, D1, idx)
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(A, sa, B, sb, D2, idx)
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(0)
    assert np.array_equal(_bits(D1), _bits(D2))


def _masked(G, max_m, N, K, mm, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((G, max_m, K)) * np.exp2(rng.integers(-6, 6, (G, max_m, 1)))).astype(np.float32)
    A, SA = _quant_act(x)
    b = (rng.standard_normal((G, N, K)) / np.sqrt(K)).astype(np.float32)
    B, SB = _quant_w(b)
    return A, SA, B, SB


@pytest.mark.parametrize("mm,max_m,N,K,cus", [([64, 0, 17, 40], 64, 128, 256, 0),
                                              ([256, 1, 129, 0, 200, 255], 256, 272, 512, 0),
                                              ([300, 7, 0, 129], 300, 400, 640, 2)])
def test_masked_ue8m0_matches_oracle(mm, max_m, N, K, cus):
    G = len(mm)
    A, SA, B, SB = _masked(G, max_m, N, K, mm, seed=max_m + N)
    mm = np.array(mm, np.int32)
    D = torch.full((G, max_m, N), -1, dtype=torch.int16, device=DEV)
    dg.dg_set_num_cus(cus)
    try:
        dg.dg_m_grouped_fp8_gemm_nt_masked_ue8m0(A, SA, B, SB, D, _t(mm))
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(0)
    got = _bits(D)
    ref = oracle.grouped_masked_ue8m0(A.cpu().numpy(), SA.cpu().numpy(), B.cpu().numpy(), SB.cpu().numpy(), mm,
                                      np.full(got.shape, SENTINEL, np.uint16))
    for g in range(G):
        m = min(max(int(mm[g]), 0), max_m)
        assert np.all(got[g, m:] == SENTINEL), f"expert {g} rows past masked_m"
        if m:
            assert_close(got[g, :m], ref[g, :m], f"masked ue8m0 expert {g}")
    # the fp32-scale kernel fed the same powers of two: bit-identical
    kb = K // 128
    D2 = torch.full((G, max_m, N), -1, dtype=torch.int16, device=DEV)
    dg.dg_m_grouped_fp8_gemm_nt_masked(A, _t(_decode_act(SA.cpu().numpy(), kb)), B,
                                       _t(ue8m0_value(unpack_k(SB.cpu().numpy(), kb))), D2, _t(mm))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(D2), got)


def test_masked_ue8m0_graph_replay_with_device_side_counts():
    G, max_m, N, K = 4, 128, 272, 512
    A, SA, B, SB = _masked(G, max_m, N, K, None, seed=5)
    MM = _t(np.array([128, 0, 0, 0], np.int32))
    D = torch.full((G, max_m, N), -1, dtype=torch.int16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dg.dg_m_grouped_fp8_gemm_nt_masked_ue8m0(A, SA, B, SB, D, MM, stream=s)
    torch.cuda.synchronize()
    a, sa, b, sb = A.cpu().numpy(), SA.cpu().numpy(), B.cpu().numpy(), SB.cpu().numpy()
    for counts in ([128, 0, 0, 0], [1, 127, 64, 0], [0, 0, 0, 128], [5, 6, 7, 8]):
        MM.copy_(torch.tensor(counts, dtype=torch.int32))
        D.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(D)
        ref = oracle.grouped_masked_ue8m0(a, sa, b, sb, np.array(counts), np.full(got.shape, SENTINEL, np.uint16))
        assert np.array_equal(got == SENTINEL, ref == SENTINEL), counts
        for e in range(G):
            if counts[e]:
                assert_close(got[e, :counts[e]], ref[e, :counts[e]], f"replay {counts} expert {e}")


@pytest.mark.timeout(600)
def test_masked_ue8m0_full_size_sampled_experts():
    # the masked decode configuration (32 experts x 256 rows, N=4096, K=7168)
    c = workloads.CONFIGS["masked"][0]
    G, max_m, N, K = c["G"], c["max_m"], c["N"], c["K"]
    w = workloads.masked(G, max_m, N, K, c["seed"])
    X = torch.zeros((G * max_m, K), dtype=torch.float32, device=DEV)
    X[torch.from_numpy(w["rows"]).to(DEV)] = _t(w["a"])
    X = X.view(G, max_m, K)
    A = torch.empty((G, max_m, K), dtype=torch.uint8, device=DEV)
    SA = torch.empty((G, _kw(K), max_m), dtype=torch.int32, device=DEV)
    dg.dg_quant_1x128_ue8m0(X, A, SA)
    Bf = _t(w["b"])
    B = torch.empty((G, N, K), dtype=torch.uint8, device=DEV)
    SB = torch.empty((G, (N + 127) // 128, _kw(K)), dtype=torch.int32, device=DEV)
    dg.dg_quant_128x128_ue8m0(Bf, B, SB)
    del Bf, X
    mm = w["masked_m"]
    D = torch.full((G, max_m, N), -1, dtype=torch.int16, device=DEV)
    dg.dg_m_grouped_fp8_gemm_nt_masked_ue8m0(A, SA, B, SB, D, _t(mm), expected_m=128)
    torch.cuda.synchronize()
    got = _bits(D)
    for e in (0, int(np.argmax(mm)), G - 1):
        m = int(mm[e])
        assert np.all(got[e, m:] == SENTINEL)
        if m:
            ref = oracle.gemm_nt_ue8m0(A[e, :m].cpu().numpy(), SA[e, :, :m].cpu().numpy(), B[e].cpu().numpy(),
                                       SB[e].cpu().numpy())
            assert_close(got[e, :m], ref, f"full-size masked ue8m0 expert {e}")
