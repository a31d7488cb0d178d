"""The contiguous layout's precondition (Lesson 13, Fig. 13-3; deep-dive
blog, section 3: expert segments padded to the 128-row M alignment), checked
on request: with DG_CHECK_LAYOUT set, a valid layout runs and matches the
oracle, and an aligned 128-row block holding rows of two experts is rejected
with DG_ERR_INVALID_ARG before anything is launched; without it the same
layout runs with the documented reading (the block's expert is the largest
valid index among its rows; only rows tagged with it are written)."""

import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import SENTINEL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _case(seed):
    counts, N, K = [130, 5, 300], 272, 512
    w = workloads.contiguous(3, N, K, seed, counts=counts)
    qa, sa = oracle.quant_1x128(w["a"])
    qa, sa = workloads.place_rows(qa, sa, w["rows"], w["m_total"])
    # every row quantised (padding rows too), so a mixed block has finite inputs
    rng = np.random.default_rng(seed)
    qfull, sfull = oracle.quant_1x128(rng.standard_normal((w["m_total"], K)).astype(np.float32))
    pad = w["m_indices"] < 0
    qa[pad], sa[:, pad] = qfull[pad], sfull[:, pad]
    qb, sb = oracle.quant_128x128(w["b"])
    return w, qa, sa, qb, sb


def _run(w, qa, sa, qb, sb, idx):
    D = torch.full((w["m_total"], qb.shape[1]), -1, dtype=torch.int16, device=DEV)
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(idx))
    torch.cuda.synchronize()
    return D.view(torch.int16).cpu().numpy().view(np.uint16)


def test_layout_check_accepts_a_padded_layout():
    w, qa, sa, qb, sb = _case(1)
    os.environ["DG_CHECK_LAYOUT"] = "1"
    try:
        got = _run(w, qa, sa, qb, sb, w["m_indices"])
    finally:
        del os.environ["DG_CHECK_LAYOUT"]
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, w["m_indices"], np.full(got.shape, SENTINEL, np.uint16))
    pad = w["m_indices"] < 0
    assert np.array_equal(got[pad], ref[pad])
    assert_close(got[~pad], ref[~pad], "checked layout")


def test_layout_check_rejects_a_block_with_two_experts():
    w, qa, sa, qb, sb = _case(2)
    idx = w["m_indices"].copy()
    # expert 0 has 130 rows: rows 128..129 share block 1 with padding; tag two
    # padding rows of that block with expert 1
    idx[200:202] = 1
    os.environ["DG_CHECK_LAYOUT"] = "1"
    try:
        D = torch.full((w["m_total"], qb.shape[1]), -1, dtype=torch.int16, device=DEV)
        with pytest.raises(dg.DGError) as ei:
            dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(idx))
        assert ei.value.code == dg.DG_ERR_INVALID_ARG and "128" in str(ei.value)
        torch.cuda.synchronize()
        assert bool((D == -1).all())
    finally:
        del os.environ["DG_CHECK_LAYOUT"]
    # unchecked: block 1 belongs to its largest valid index (1); its rows tagged
    # 1 are computed with expert 1's weights, its rows tagged 0 are not written
    got = _run(w, qa, sa, qb, sb, idx)
    keep = idx.copy()
    keep[128:256][keep[128:256] == 0] = -1
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, keep, np.full(got.shape, SENTINEL, np.uint16))
    untouched = keep < 0
    assert np.array_equal(got[untouched], ref[untouched])
    assert_close(got[~untouched], ref[~untouched], "unchecked mixed block")
