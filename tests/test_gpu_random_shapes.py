"""Seeded random shapes over every GEMM entry point and planner branch,
against the oracle.

Each case draws an entry point (dense fp8, accumulating fp32, UE8M0 and bf16
dense; contiguous and masked, with fp32 or UE8M0 scales), a ragged shape, a
CU cap and a forced plan (tile kernel, skinny configuration with a K split,
small row chunks), so that combinations the hand-written cases do not list
still meet the same bars: bf16 results within the per-element tolerance,
fp32 results within the derived bound and the per-element rule, and rows the
call must not write left bit-exact untouched."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import SENTINEL, acc_tolerance, assert_close, assert_f32_rule, masked_layout

pytestmark = pytest.mark.gpu
DEV = "cuda"
FORMS = ("dense", "acc", "ue8m0", "bf16", "contiguous", "masked", "contiguous_ue8m0", "masked_ue8m0")
SKINNY = ("64x16x{}x4", "64x16x{}x8", "64x32x{}x4", "64x32x{}x6", "128x16x{}x6", "128x32x{}x4")
N_CASES = 160


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _case(i):
    rng = np.random.default_rng(9000 + i)
    form = FORMS[i % len(FORMS)]
    c = dict(form=form, seed=9000 + i, cus=int(rng.choice([0, 0, 1, 5, 37, 111])), force=None)
    c["N"] = 16 * int(rng.integers(1, 50))
    c["K"] = 64 * int(rng.integers(1, 21)) if form == "bf16" else 128 * int(rng.integers(1, 11))
    if form in ("dense", "acc", "ue8m0", "bf16"):
        c["M"] = int(rng.integers(1, 129)) if rng.random() < 0.5 else int(rng.integers(129, 700))
        # the skinny kernel takes up to 2048 rows: half the cases past 128
        # rows go there, the other half to the tile kernels
        if form != "bf16" and (c["M"] <= 128 or (c["M"] <= 2048 and rng.random() < 0.5)):
            if rng.random() < 0.8:
                c["force"] = "skinny=" + str(rng.choice(SKINNY)).format(int(rng.integers(1, 5)))
        else:
            opts = [None, "kernel=wide", "kernel=persistent"] + (["chunk_rows=256"] if c["M"] > 256 else [])
            c["force"] = opts[int(rng.integers(0, len(opts)))]
    elif form.startswith("contiguous"):
        c["counts"] = [int(x) for x in rng.integers(0, 400, int(rng.integers(1, 7)))]
        c["force"] = [None, "kernel=wide", "kernel=persistent"][int(rng.integers(0, 3))]
    else:
        c["G"] = int(rng.integers(1, 7))
        c["max_m"] = int(rng.choice([16, 64, 128, 200, 256, 300]))
        c["masked_m"] = [int(x) for x in rng.integers(0, c["max_m"] + 1, c["G"])]
    return c


def _ws(op, rows, N, K, G=1):
    n = dg.dg_get_workspace_size(op, rows, N, K, G)
    return torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV) if n else None


def _dense(c):
    M, N, K, form = c["M"], c["N"], c["K"], c["form"]
    if form == "bf16":
        a, b = workloads.dense_bf16(M, N, K, c["seed"])
        D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
        dg.dg_bf16_gemm_nt(_t(a), _t(b), D, _ws(dg.DG_OP_BF16_GEMM_NT, M, N, K))
        assert_close(_bits(D), oracle.gemm_bf16_nt(a, b), f"bf16 {c}")
        return
    a32, b32 = workloads.dense(M, N, K, c["seed"])
    if form == "ue8m0":
        qa, _, pa = oracle.quant_1x128_ue8m0(a32)
        qb, _, pb = oracle.quant_128x128_ue8m0(b32)
        D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
        dg.dg_fp8_gemm_nt_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D, _ws(dg.DG_OP_GEMM_NT_UE8M0, M, N, K))
        assert_close(_bits(D), oracle.gemm_nt_ue8m0(qa, pa, qb, pb), f"ue8m0 {c}")
        return
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    if form == "dense":
        D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
        dg.dg_fp8_gemm_nt(_t(qa), _t(sa), _t(qb), _t(sb), D, _ws(dg.DG_OP_GEMM_NT, M, N, K))
        assert_close(_bits(D), oracle.gemm_nt(qa, sa, qb, sb), f"dense {c}")
        return
    cm = np.random.default_rng(c["seed"] + 1).standard_normal((M, N)).astype(np.float32)
    D = _t(cm)  # accumulated in place
    dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), D, D, _ws(dg.DG_OP_GEMM_NT, M, N, K))
    torch.cuda.synchronize()
    got = D.cpu().numpy().astype(np.float64)
    ref = oracle.gemm_nt_c(qa, sa, qb, sb, cm).astype(np.float64)
    tol = acc_tolerance(qa, sa, qb, sb, cm)
    assert np.all(np.abs(got - ref) <= tol), f"acc {c}: {int((np.abs(got - ref) > tol).sum())} beyond the bound"
    assert_f32_rule(got, ref, f"acc {c}")


def _contiguous(c):
    counts, N, K, ue = c["counts"], c["N"], c["K"], c["form"].endswith("ue8m0")
    G = len(counts)
    w = workloads.contiguous(G, N, K, c["seed"], counts=counts)
    m_total = w["m_total"]
    if m_total == 0:
        return
    D = torch.full((m_total, N), -1, dtype=torch.int16, device=DEV)
    init = np.full((m_total, N), SENTINEL, np.uint16)
    if ue:
        qv, _, pv = oracle.quant_1x128_ue8m0(w["a"]) if w["rows"].size else (None, None, None)
        qa = np.full((m_total, K), workloads.TRAP_CODE, np.uint8)
        pa = np.zeros(((K // 128 + 3) // 4, m_total), np.int32)
        if w["rows"].size:
            qa[w["rows"]], pa[:, w["rows"]] = qv, pv
        qw = [oracle.quant_128x128_ue8m0(w["b"][g]) for g in range(G)]
        qb = np.stack([x[0] for x in qw])
        pb = np.stack([x[2] for x in qw])
        dg.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D, _t(w["m_indices"]))
        ref = oracle.grouped_contiguous_ue8m0(qa, pa, qb, pb, w["m_indices"], init)
    else:
        if w["rows"].size:
            qv, sv = oracle.quant_1x128(w["a"])
        else:
            qv, sv = np.zeros((0, K), np.uint8), np.zeros((K // 128, 0), np.float32)
        qa, sa = workloads.place_rows(qv, sv, w["rows"], m_total)
        qb, sb = oracle.quant_128x128(w["b"])
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(w["m_indices"]))
        ref = oracle.grouped_contiguous(qa, sa, qb, sb, w["m_indices"], init)
    got = _bits(D)
    pad = w["m_indices"] < 0
    assert np.array_equal(got[pad], ref[pad]), f"padding rows written {c}"
    if (~pad).any():
        assert_close(got[~pad], ref[~pad], f"contiguous {c}")


def _masked(c):
    G, max_m, N, K, ue = c["G"], c["max_m"], c["N"], c["K"], c["form"].endswith("ue8m0")
    w = workloads.masked(G, max_m, N, K, c["seed"], masked_m=c["masked_m"])
    D = torch.full((G, max_m, N), -1, dtype=torch.int16, device=DEV)
    init = np.full((G, max_m, N), SENTINEL, np.uint16)
    KW = (K // 128 + 3) // 4
    if ue:
        qa = np.full((G * max_m, K), workloads.TRAP_CODE, np.uint8)
        pa = np.zeros((KW, G * max_m), np.int32)
        if w["rows"].size:
            qv, _, pv = oracle.quant_1x128_ue8m0(w["a"])
            qa[w["rows"]], pa[:, w["rows"]] = qv, pv
        qa = qa.reshape(G, max_m, K)
        pa = np.ascontiguousarray(pa.reshape(KW, G, max_m).transpose(1, 0, 2))
        qw = [oracle.quant_128x128_ue8m0(w["b"][g]) for g in range(G)]
        qb = np.stack([x[0] for x in qw])
        pb = np.stack([x[2] for x in qw])
        dg.dg_m_grouped_fp8_gemm_nt_masked_ue8m0(_t(qa), _t(pa), _t(qb), _t(pb), D, _t(w["masked_m"]))
        ref = oracle.grouped_masked_ue8m0(qa, pa, qb, pb, w["masked_m"], init)
    else:
        if w["rows"].size:
            qv, sv = oracle.quant_1x128(w["a"])
        else:
            qv, sv = np.zeros((0, K), np.uint8), np.zeros((K // 128, 0), np.float32)
        qa, sa = masked_layout(qv, sv, w["rows"], G, max_m)
        qb, sb = oracle.quant_128x128(w["b"])
        dg.dg_m_grouped_fp8_gemm_nt_masked(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(w["masked_m"]))
        ref = oracle.grouped_masked(qa, sa, qb, sb, w["masked_m"], init)
    got = _bits(D)
    valid = np.zeros((G, max_m), bool)
    for g, m in enumerate(w["masked_m"]):
        valid[g, :min(max(int(m), 0), max_m)] = True
    assert np.array_equal(got[~valid], ref[~valid]), f"rows past masked_m written {c}"
    if valid.any():
        assert_close(got[valid], ref[valid], f"masked {c}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i, monkeypatch):
    c = _case(i)
    if c["force"]:
        monkeypatch.setenv("DG_FORCE_CONFIG", c["force"])
    print(f"case {i}: {c}", flush=True)
    dg.dg_set_num_cus(c["cus"])
    try:
        if c["form"] in ("dense", "acc", "ue8m0", "bf16"):
            _dense(c)
        elif c["form"].startswith("contiguous"):
            _contiguous(c)
        else:
            _masked(c)
    finally:
        dg.dg_set_num_cus(0)
