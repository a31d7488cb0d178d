"""Full-size parity at the benchmark's shapes and launch configuration.

Every configuration runs exactly as bench.py runs it: fp32 sources drawn by
moe_grouped_matmul_amd.workloads, quantised on the GPU (dg_quant_1x128 /
dg_quant_128x128), then the GEMM.  The oracle cannot afford whole outputs at
these sizes, so it quantises, from the same fp32 sources, only sampled rows of
A and sampled 128-row blocks of B.  The GPU bytes and scales of exactly those
rows/blocks must equal the oracle's (bit-exact), and the GEMM outputs at
(sampled rows) x (sampled column blocks) must meet the element tolerance,
with rms(ref) taken over the sample.  Rows the operation must not write
(contiguous padding, masked-off rows) are checked over the whole output.
"""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import SENTINEL, assert_close

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

DEV = torch.device("cuda:0")


def _gpu_quant_a(a32):
    A32 = torch.from_numpy(a32).to(DEV)
    R, K = A32.shape
    q = torch.empty((R, K), dtype=torch.uint8, device=DEV)
    s = torch.empty((K // 128, R), dtype=torch.float32, device=DEV)
    if R:
        dg.dg_quant_1x128(A32, q, s)
    return q, s


def _gpu_quant_b(b32):
    B32 = torch.from_numpy(b32).to(DEV)
    q = torch.empty(B32.shape, dtype=torch.uint8, device=DEV)
    s = torch.empty(B32.shape[:-2] + ((B32.shape[-2] + 127) // 128, B32.shape[-1] // 128), dtype=torch.float32,
                    device=DEV)
    dg.dg_quant_128x128(B32, q, s)
    del B32
    return q, s


def _sample_rows(n, k, rng):
    if n <= k:
        return np.arange(n)
    pick = {0, n // 2, n - 1}
    while len(pick) < k:
        pick.add(int(rng.integers(0, n)))
    return np.array(sorted(pick))


def _col_blocks(N):
    nb = (N + 127) // 128
    return sorted({0, nb // 2, nb - 1})


def _check_sample(a32_rows, gq_rows, gs_rows, b32, gqb, gsb, got_rows, N, what):
    """a32_rows: fp32 [r, K]; gq_rows/gs_rows: GPU bytes [r, K] / scales [K/128, r] of those rows;
    b32: fp32 [N, K] of one expert; gqb/gsb: GPU bytes [N, K] / scales [NB, K/128]; got_rows: GPU D [r, N]."""
    qa, sa = oracle.quant_1x128(a32_rows)
    assert np.array_equal(gq_rows, qa), f"{what}: activation bytes differ"
    assert np.array_equal(gs_rows.view(np.uint32), sa.view(np.uint32)), f"{what}: activation scales differ"
    for b in _col_blocks(N):
        c0, c1 = 128 * b, min(128 * b + 128, N)
        qb, sb = oracle.quant_128x128(b32[c0:c1])
        assert np.array_equal(gqb[c0:c1], qb), f"{what}: weight bytes differ in block {b}"
        assert np.array_equal(gsb[b:b + 1].view(np.uint32), sb.view(np.uint32)), f"{what}: weight scale differs"
        ref = oracle.gemm_nt(qa, sa, qb, sb)
        assert_close(got_rows[:, c0:c1], ref, f"{what} columns {c0}:{c1}")


DENSE = workloads.CONFIGS["dense_small"] + workloads.CONFIGS["dense_sweep"] + workloads.CONFIGS["dense_large"]


@pytest.mark.parametrize("shape", DENSE, ids=lambda s: f"{s['M']}x{s['N']}x{s['K']}-seed{s['seed']}")
def test_dense_full_size(shape):
    M, N, K, seed = shape["M"], shape["N"], shape["K"], shape["seed"]
    print(f"dense {M}x{N}x{K} seed {seed}", flush=True)
    a32, b32 = workloads.dense(M, N, K, seed)
    qa, sa = _gpu_quant_a(a32)
    qb, sb = _gpu_quant_b(b32)
    D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
    n = dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT, M, N, K, 1)
    ws = torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV) if n else None
    dg.dg_fp8_gemm_nt(qa, sa, qb, sb, D, ws)
    torch.cuda.synchronize()
    rows = _sample_rows(M, 24, np.random.default_rng(seed))
    ridx = torch.from_numpy(rows).to(DEV)
    got = D.index_select(0, ridx).cpu().numpy().view(np.uint16)
    gq = qa.index_select(0, ridx).cpu().numpy()
    gs = sa.index_select(1, ridx).cpu().numpy()
    _check_sample(a32[rows], gq, gs, b32, qb.cpu().numpy(), sb.cpu().numpy(), got, N, f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("cfg", workloads.CONFIGS["contiguous"], ids=lambda c: f"G{c['G']}-{c['N']}x{c['K']}")
def test_contiguous_full_size(cfg):
    G, N, K, seed = cfg["G"], cfg["N"], cfg["K"], cfg["seed"]
    print(f"contiguous G={G} {N}x{K} seed {seed}", flush=True)
    w = workloads.contiguous(G, N, K, seed)
    m_total, rows = w["m_total"], w["rows"]
    q, s = _gpu_quant_a(w["a"])
    ridx = torch.from_numpy(rows).to(DEV)
    A8 = torch.full((m_total, K), workloads.TRAP_CODE, dtype=torch.uint8, device=DEV)
    SA = torch.full((K // 128, m_total), float("nan"), dtype=torch.float32, device=DEV)
    A8[ridx] = q
    SA[:, ridx] = s
    qb, sb = _gpu_quant_b(w["b"])
    D = torch.full((m_total, N), -1, dtype=torch.int16, device=DEV)
    idx = torch.from_numpy(w["m_indices"]).to(DEV)
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(A8, SA, qb, sb, D, idx)
    torch.cuda.synchronize()
    pad = idx < 0
    assert bool((D[pad] == -1).all()), "padding rows were written"
    qb_h, sb_h = qb.cpu().numpy(), sb.cpu().numpy()
    rng = np.random.default_rng(seed)
    start = 0
    for e in range(G):
        c = int(w["counts"][e])
        local = _sample_rows(c, 6, rng)  # row numbers inside the expert's valid rows
        pos = rows[start + local]  # positions in the padded layout
        pidx = torch.from_numpy(pos).to(DEV)
        got = D.index_select(0, pidx).cpu().numpy().view(np.uint16)
        gq = A8.index_select(0, pidx).cpu().numpy()
        gs = SA.index_select(1, pidx).cpu().numpy()
        _check_sample(w["a"][start + local], gq, gs, w["b"][e], qb_h[e], sb_h[e], got, N, f"contiguous expert {e}")
        start += c


@pytest.mark.parametrize("cfg", workloads.CONFIGS["masked"] + workloads.CONFIGS["masked_decode"],
                         ids=lambda c: f"G{c['G']}x{c['max_m']}-{c['N']}x{c['K']}")
def test_masked_full_size(cfg):
    G, max_m, N, K, seed = cfg["G"], cfg["max_m"], cfg["N"], cfg["K"], cfg["seed"]
    print(f"masked G={G} max_m={max_m} {N}x{K} seed {seed}", flush=True)
    w = workloads.masked(G, max_m, N, K, seed)
    rows = w["rows"]
    q, s = _gpu_quant_a(w["a"])
    ridx = torch.from_numpy(rows).to(DEV)
    A8 = torch.full((G * max_m, K), workloads.TRAP_CODE, dtype=torch.uint8, device=DEV)
    SAf = torch.full((K // 128, G * max_m), float("nan"), dtype=torch.float32, device=DEV)
    A8[ridx] = q
    SAf[:, ridx] = s
    A8 = A8.view(G, max_m, K)
    SA = SAf.view(K // 128, G, max_m).permute(1, 0, 2).contiguous()
    qb, sb = _gpu_quant_b(w["b"])
    D = torch.full((G, max_m, N), -1, dtype=torch.int16, device=DEV)
    mm = torch.from_numpy(w["masked_m"]).to(DEV)
    dg.dg_m_grouped_fp8_gemm_nt_masked(A8, SA, qb, sb, D, mm, expected_m=max_m // 2)
    torch.cuda.synchronize()
    valid = torch.arange(max_m, device=DEV)[None, :] < mm[:, None]
    assert bool((D[~valid] == -1).all()), "rows past masked_m were written"
    qb_h, sb_h = qb.cpu().numpy(), sb.cpu().numpy()
    rng = np.random.default_rng(seed)
    start = 0
    for g in range(G):
        m = int(w["masked_m"][g])
        if m == 0:
            continue
        local = _sample_rows(m, 4, rng)
        lidx = torch.from_numpy(local).to(DEV)
        got = D[g].index_select(0, lidx).cpu().numpy().view(np.uint16)
        gq = A8[g].index_select(0, lidx).cpu().numpy()
        gs = SA[g].index_select(1, lidx).cpu().numpy()
        _check_sample(w["a"][start + local], gq, gs, w["b"][g], qb_h[g], sb_h[g], got, N, f"masked expert {g}")
        start += m
