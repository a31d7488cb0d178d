"""The largest group count the boundary accepts (G = 1024) on every grouped
form, against the oracle: the device-side task and segment tables of the
masked, contiguous and K-grouped kernels are then at their largest.  Tiny
experts keep the oracle fast; the counts are ragged (empty experts, counts
past the capacity or negative for the masked form, which the kernel clamps)."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import SENTINEL, assert_close, assert_f32_rule, kg_tolerance, masked_layout

pytestmark = pytest.mark.gpu
DEV = "cuda"
G = 1024


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("ue", [False, True])
def test_masked_1024_experts(ue):
    max_m, N, K = 20, 32, 256
    rng = np.random.default_rng(71)
    mm = rng.integers(0, max_m + 1, G).astype(np.int32)
    mm[::97] = -3          # negative: no rows
    mm[5::101] = max_m + 7  # past the capacity: all rows
    w = workloads.masked(G, max_m, N, K, 72, masked_m=mm)
    D = torch.full((G, max_m, N), -1, dtype=torch.int16, device=DEV)
    init = np.full((G, max_m, N), SENTINEL, np.uint16)
    if ue:
        KW = (K // 128 + 3) // 4
        qa = np.full((G * max_m, K), workloads.TRAP_CODE, np.uint8)
        pa = np.zeros((KW, G * max_m), np.int32)
        qv, _, pv = oracle.quant_1x128_ue8m0(w["a"])
        qa[w["rows"]], pa[:, w["rows"]] = qv, pv
        qa = qa.reshape(G, max_m, K)
        pa = np.ascontiguousarray(pa.reshape(KW, G, max_m).transpose(1, 0, 2))
        qw = [oracle.quant_128x128_ue8m0(w["b"][g]) for g in range(G)]
        qb, pb = np.stack([x[0] for x in qw]), np.stack([x[2] for x in qw])
        dg.dg_m_grouped_fp8_gemm_nt_masked_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D, _t(mm))
        ref = oracle.grouped_masked_ue8m0(qa, pa, qb, pb, mm, init)
    else:
        qv, sv = oracle.quant_1x128(w["a"])
        qa, sa = masked_layout(qv, sv, w["rows"], G, max_m)
        qb, sb = oracle.quant_128x128(w["b"])
        dg.dg_m_grouped_fp8_gemm_nt_masked(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(mm))
        ref = oracle.grouped_masked(qa, sa, qb, sb, mm, init)
    got = _bits(D)
    valid = np.zeros((G, max_m), bool)
    for g in range(G):
        valid[g, :min(max(int(mm[g]), 0), max_m)] = True
    assert np.array_equal(got[~valid], ref[~valid]), "rows past masked_m written"
    assert_close(got[valid], ref[valid], f"masked G={G} ue8m0={ue}")


def test_contiguous_1024_experts():
    N, K = 32, 128
    rng = np.random.default_rng(73)
    counts = rng.integers(0, 4, G)
    w = workloads.contiguous(G, N, K, 74, counts=counts)
    qv, sv = oracle.quant_1x128(w["a"])
    qa, sa = workloads.place_rows(qv, sv, w["rows"], w["m_total"])
    qb, sb = oracle.quant_128x128(w["b"])
    D = torch.full((w["m_total"], N), -1, dtype=torch.int16, device=DEV)
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(w["m_indices"]))
    got = _bits(D)
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, w["m_indices"], np.full(got.shape, SENTINEL, np.uint16))
    pad = w["m_indices"] < 0
    assert np.array_equal(got[pad], ref[pad]), "padding rows written"
    assert_close(got[~pad], ref[~pad], f"contiguous G={G}")


def test_k_grouped_1024_groups():
    M, N = 64, 48
    w = workloads.k_grouped(G, M, N, 75, max_tokens=130)
    qa, sa = oracle.quant_1x128(w["a"])
    qb, sb = oracle.quant_1x128(w["b"])
    c = (np.random.default_rng(76).standard_normal((G, M, N)) * 10.0).astype(np.float32)
    D = _t(c)  # in place
    dg.dg_k_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, D, _t(w["ks"]))
    torch.cuda.synchronize()
    got = D.cpu().numpy()
    ref = oracle.k_grouped_contiguous(qa, sa, qb, sb, w["ks"], c)
    tol = kg_tolerance(qa, sa, qb, sb, w["ks"], c)
    assert np.all(np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= tol), "outside the arithmetic bound"
    assert_f32_rule(got, ref, f"k-grouped G={G}")
