"""K-grouped contiguous FP8 GEMM (dg_k_grouped_fp8_gemm_nt_contiguous,
D[g] = C[g] + A[:, seg g] . B[:, seg g]^T in fp32) against the oracle
(oracle.k_grouped_contiguous): ragged M and N, empty groups, one and many
groups, an unused K tail, C given / absent / in place, many tiles per
workgroup on 256 x 128 and 256 x 256 tiles, the kernel's documented handling of lengths that are negative,
unaligned or run past K, graph replay with device-side length changes,
integer inputs bit-exact, and the two weight-gradient shapes at full size on
sampled rows and columns."""

import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import assert_f32_rule, kg_tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _case(G, M, N, seed, counts=None, max_tokens=700):
    w = workloads.k_grouped(G, M, N, seed, max_tokens=max_tokens, counts=counts)
    qa, sa = oracle.quant_1x128(w["a"])
    qb, sb = oracle.quant_1x128(w["b"])
    rng = np.random.default_rng(seed + 1)
    c = (rng.standard_normal((G, M, N)) * 10.0).astype(np.float32)
    return qa, sa, qb, sb, w["ks"], c


def _check(got, qa, sa, qb, sb, ks, c, what):
    ref = oracle.k_grouped_contiguous(qa, sa, qb, sb, ks, c)
    tol = kg_tolerance(qa, sa, qb, sb, ks, c)
    bad = ~(np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= tol)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the bound, e.g. " \
                          f"{[(tuple(i), float(got[tuple(i)]), float(ref[tuple(i)])) for i in np.argwhere(bad)[:3]]}"
    # the per-element acceptance rule on top of the arithmetic ceiling above
    assert_f32_rule(got, ref, what)


def _run(qa, sa, qb, sb, ks, C, D):
    dg.dg_k_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), C, D, _t(ks.astype(np.int32)))
    torch.cuda.synchronize()


CASES = [
    # G, M, N, counts (None: drawn), max_tokens
    (1, 256, 128, [384], 0),
    (2, 300, 272, None, 700),
    (4, 64, 16, [0, 130, 0, 1], 0),
    (3, 513, 400, [1000, 0, 257], 0),
    (8, 200, 1040, None, 900),
    (40, 130, 144, None, 300),
]


@pytest.mark.parametrize("G,M,N,counts,maxt", CASES)
@pytest.mark.parametrize("mode", ["c", "none", "inplace"])
def test_k_grouped_matches_oracle(G, M, N, counts, maxt, mode):
    qa, sa, qb, sb, ks, c = _case(G, M, N, seed=G * 1000 + M + N, counts=counts, max_tokens=maxt or 700)
    C = None if mode == "none" else _t(c)
    D = C if mode == "inplace" else torch.full((G, M, N), float("nan"), dtype=torch.float32, device=DEV)
    _run(qa, sa, qb, sb, ks, C, D)
    _check(D.cpu().numpy(), qa, sa, qb, sb, ks, None if mode == "none" else c, f"k-grouped G={G} {M}x{N} {mode}")


# (cus, G, M, N, counts): 256 x 256 tiles (the wide kernel) once the tiles of
# all groups fill whole rounds of the capped CUs: ragged M and N, an empty
# group, several groups and tiles per workgroup
WIDE = [(1, 1, 256, 256, [384]), (2, 2, 300, 272, None), (3, 3, 513, 400, [1000, 0, 257]), (4, 8, 256, 1040, None)]


@pytest.mark.parametrize("cus,G,M,N,counts", WIDE)
@pytest.mark.parametrize("mode", ["c", "none", "inplace"])
def test_k_grouped_wide_tiles(capfd, cus, G, M, N, counts, mode):
    dg.dg_set_num_cus(cus)
    os.environ["DG_PRINT_CONFIGS"] = "1"
    try:
        qa, sa, qb, sb, ks, c = _case(G, M, N, seed=cus * 100 + G + M, counts=counts, max_tokens=700)
        C = None if mode == "none" else _t(c)
        D = C if mode == "inplace" else torch.full((G, M, N), float("nan"), dtype=torch.float32, device=DEV)
        capfd.readouterr()
        _run(qa, sa, qb, sb, ks, C, D)
        assert "kernel=wide" in capfd.readouterr().err
    finally:
        del os.environ["DG_PRINT_CONFIGS"]
        dg.dg_set_num_cus(0)
    _check(D.cpu().numpy(), qa, sa, qb, sb, ks, None if mode == "none" else c,
           f"k-grouped wide G={G} {M}x{N} {mode} on {cus} CUs")


def test_k_grouped_wide_integer_inputs_bit_exact():
    rng = np.random.default_rng(15)
    G, M, N, ks = 3, 300, 272, np.array([256, 0, 384], np.int32)
    K = int(ks.sum())
    qa = oracle.encode_e4m3(rng.integers(-10, 10, (M, K)).astype(np.float32))
    qb = oracle.encode_e4m3(rng.integers(-10, 10, (N, K)).astype(np.float32))
    sa = np.ones((K // 128, M), np.float32)
    sb = np.ones((K // 128, N), np.float32)
    c = rng.integers(-5000, 5000, (G, M, N)).astype(np.float32)
    dg.dg_set_num_cus(2)
    try:
        D = _t(c)  # in place
        _run(qa, sa, qb, sb, ks, D, D)
    finally:
        dg.dg_set_num_cus(0)
    assert np.array_equal(D.cpu().numpy(), oracle.k_grouped_contiguous(qa, sa, qb, sb, ks, c))


@pytest.mark.parametrize("cus", [1, 7, 9])  # 1 and 7: 256 x 256 tiles; 9: 256 x 128 tiles
def test_k_grouped_many_tiles_per_workgroup(cus):
    dg.dg_set_num_cus(cus)
    try:
        qa, sa, qb, sb, ks, c = _case(5, 700, 304, seed=cus, max_tokens=600)
        D = torch.empty((5, 700, 304), dtype=torch.float32, device=DEV)
        _run(qa, sa, qb, sb, ks, _t(c), D)
    finally:
        dg.dg_set_num_cus(0)
    _check(D.cpu().numpy(), qa, sa, qb, sb, ks, c, f"k-grouped on {cus} CUs")


def test_k_grouped_unused_k_tail():
    # the segments cover the first 512 of 896 K positions; the rest belong to no group
    qa, sa, qb, sb, ks, c = _case(2, 260, 144, seed=11, counts=[300, 150])
    K = qa.shape[1]
    pad = 384
    rng = np.random.default_rng(12)
    qa2 = np.concatenate([qa, rng.integers(0, 0x7E, (qa.shape[0], pad), dtype=np.uint8)], axis=1)
    qb2 = np.concatenate([qb, rng.integers(0, 0x7E, (qb.shape[0], pad), dtype=np.uint8)], axis=1)
    sa2 = np.concatenate([sa, np.full((pad // 128, sa.shape[1]), 3.0, np.float32)])
    sb2 = np.concatenate([sb, np.full((pad // 128, sb.shape[1]), 3.0, np.float32)])
    assert qa2.shape[1] == K + pad
    D = torch.empty((2, 260, 144), dtype=torch.float32, device=DEV)
    _run(qa2, sa2, qb2, sb2, ks, _t(c), D)
    _check(D.cpu().numpy(), qa2, sa2, qb2, sb2, ks, c, "unused K tail")


def test_k_grouped_length_rules():
    # negative lengths count as 0, lengths round down to multiples of 128, and
    # blocks past K are dropped (the header's rule); compared with the oracle
    # on the lengths that rule yields
    qa, sa, qb, sb, ks, c = _case(4, 200, 128, seed=13, counts=[256, 256, 128, 0])
    K = qa.shape[1]
    raw = np.array([-5, 300, 200, 4096], np.int32)
    eff, lo = [], 0
    for k in raw:
        n = max(int(k), 0) // 128 * 128
        n = min(n, K - lo)
        eff.append(n)
        lo += n
    D = torch.empty((4, 200, 128), dtype=torch.float32, device=DEV)
    dg.dg_k_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), _t(c), D, _t(raw))
    torch.cuda.synchronize()
    _check(D.cpu().numpy(), qa, sa, qb, sb, np.array(eff), c, "length rules")


def test_k_grouped_integer_inputs_bit_exact():
    rng = np.random.default_rng(14)
    G, M, N, ks = 3, 300, 160, np.array([256, 0, 384], np.int32)
    K = int(ks.sum())
    qa = oracle.encode_e4m3(rng.integers(-10, 10, (M, K)).astype(np.float32))
    qb = oracle.encode_e4m3(rng.integers(-10, 10, (N, K)).astype(np.float32))
    sa = np.ones((K // 128, M), np.float32)
    sb = np.ones((K // 128, N), np.float32)
    c = rng.integers(-5000, 5000, (G, M, N)).astype(np.float32)
    ref = oracle.k_grouped_contiguous(qa, sa, qb, sb, ks, c)
    D = torch.empty((G, M, N), dtype=torch.float32, device=DEV)
    _run(qa, sa, qb, sb, ks, _t(c), D)
    assert np.array_equal(D.cpu().numpy(), ref)


def test_k_grouped_graph_replay_with_device_lengths():
    # the kernel reads ks on the device: a captured call follows changes of
    # ks between replays (same total K)
    qa, sa, qb, sb, ks, c = _case(3, 256, 256, seed=15, counts=[256, 256, 256])
    A, SA, B, SB = _t(qa), _t(sa), _t(qb), _t(sb)
    KS = _t(ks.astype(np.int32))
    D = torch.empty((3, 256, 256), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dg.dg_k_grouped_fp8_gemm_nt_contiguous(A, SA, B, SB, None, D, KS, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dg.dg_k_grouped_fp8_gemm_nt_contiguous(A, SA, B, SB, None, D, KS, stream=s)
    torch.cuda.synchronize()
    for lengths in ([256, 256, 256], [512, 0, 256], [0, 128, 640], [768, 0, 0]):
        KS.copy_(torch.tensor(lengths, dtype=torch.int32))
        D.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(D.cpu().numpy(), qa, sa, qb, sb, np.array(lengths), None, f"graph replay {lengths}")


# ---- full size, bench launch configuration, sampled rows/columns

def _sample(n, k, rng):
    pick = {0, n // 2, n - 1}
    while len(pick) < k:
        pick.add(int(rng.integers(0, n)))
    return np.array(sorted(pick))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", workloads.CONFIGS["k_grouped"], ids=lambda s: f"G{s['G']}-{s['M']}x{s['N']}")
def test_k_grouped_full_size(shape):
    G, M, N, seed = shape["G"], shape["M"], shape["N"], shape["seed"]
    w = workloads.k_grouped(G, M, N, seed)
    ks = w["ks"]
    K = int(ks.sum())

    def gq(x):
        X = torch.from_numpy(x).to(DEV)
        q = torch.empty(X.shape, dtype=torch.uint8, device=DEV)
        s = torch.empty((K // 128, X.shape[0]), dtype=torch.float32, device=DEV)
        dg.dg_quant_1x128(X, q, s)
        del X
        return q, s

    A, SA = gq(w["a"])
    B, SB = gq(w["b"])
    D = torch.empty((G, M, N), dtype=torch.float32, device=DEV)
    dg.dg_k_grouped_fp8_gemm_nt_contiguous(A, SA, B, SB, None, D, _t(ks))
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = _sample(M, 12, rng)
    cols = _sample(N, 12, rng)
    qa, sa = oracle.quant_1x128(w["a"][rows])
    qb, sb = oracle.quant_1x128(w["b"][cols])
    assert np.array_equal(A[torch.from_numpy(rows).to(DEV)].cpu().numpy(), qa)
    assert np.array_equal(SA[:, torch.from_numpy(rows).to(DEV)].cpu().numpy().view(np.uint32), sa.view(np.uint32))
    assert np.array_equal(B[torch.from_numpy(cols).to(DEV)].cpu().numpy(), qb)
    assert np.array_equal(SB[:, torch.from_numpy(cols).to(DEV)].cpu().numpy().view(np.uint32), sb.view(np.uint32))
    got = D.cpu().numpy()[:, rows][:, :, cols]
    _check(got, qa, sa, qb, sb, ks, None, f"full size G={G} {M}x{N}x{K}")
    assert np.isfinite(D.cpu().numpy()).all()
