"""Scale indexing, checked bit-exactly on every GEMM kernel path.

Integer e4m3 codes in [-4, 4] with power-of-two scales that vary per row and
K block (alpha) and per column block and K block (beta; per column and K
block for the K-grouped form, whose weights carry 1x128 scales).  Every MFMA
partial is an integer below 2^11, every scale product a power of two in
[2^-4, 2^4], and every running sum a multiple of 2^-4 of magnitude at most
2^20 (K <= 4096), so the fp32 arithmetic of the kernels is exact and their
results must equal the oracle's bit for bit (bf16 outputs: both round the same exact value to nearest even).
A scale read from the wrong row, column block or K block changes the result
by at least one unit of 2^-4 and fails the comparison (Lesson 13, Fig. 13-1:
alpha per row and 1x128 K group, beta per 128x128 block)."""

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _codes(rng, rows, K):
    return oracle.encode_e4m3(rng.integers(-4, 5, (rows, K)).astype(np.float32))


def _pow2(rng, shape):
    return np.ldexp(np.float32(1.0), rng.integers(-2, 3, shape)).astype(np.float32)


def _plan(op, rows, N, K, G=1):
    return dg.dg_describe_plan(op, rows, N, K, G)


class _Cus:
    def __init__(self, n):
        self.n = n

    def __enter__(self):
        dg.dg_set_num_cus(self.n)

    def __exit__(self, *a):
        dg.dg_set_num_cus(0)


def _ws(op, M, N, K):
    n = dg.dg_get_workspace_size(op, M, N, K, 1)
    return torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV) if n else None


# (cus, M, N, K, kernel the planner is expected to take)
DENSE = [(0, 64, 272, 512, "skinny"), (0, 100, 2112, 4096, "skinny"), (0, 300, 400, 512, "skinny"),
         (0, 333, 1536, 4096, "skinny"), (0, 320, 7168, 1024, "skinny"), (0, 384, 4096, 2048, "skinny"),
         (0, 700, 1536, 1024, "skinny"), (0, 2100, 400, 512, "persistent"), (5, 1000, 528, 640, "persistent"), (4, 512, 496, 512, "wide"),
         (2, 300, 608, 384, "wide")]


@pytest.mark.parametrize("cus,M,N,K,kernel", DENSE)
def test_dense_varying_power_of_two_scales_bit_exact(cus, M, N, K, kernel):
    rng = np.random.default_rng(M * 7 + N)
    qa, qb = _codes(rng, M, K), _codes(rng, N, K)
    sa = _pow2(rng, (K // 128, M))
    sb = _pow2(rng, ((N + 127) // 128, K // 128))
    with _Cus(cus):
        assert f"kernel={kernel}" in _plan(dg.DG_OP_GEMM_NT, M, N, K)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        dg.dg_fp8_gemm_nt(_t(qa), _t(sa), _t(qb), _t(sb), D, _ws(dg.DG_OP_GEMM_NT, M, N, K))
        torch.cuda.synchronize()
    got = D.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.gemm_nt(qa, sa, qb, sb))


@pytest.mark.parametrize("cus,M,N,K,kernel", DENSE)
def test_acc_varying_power_of_two_scales_bit_exact(cus, M, N, K, kernel):
    rng = np.random.default_rng(M * 11 + N)
    qa, qb = _codes(rng, M, K), _codes(rng, N, K)
    sa = _pow2(rng, (K // 128, M))
    sb = _pow2(rng, ((N + 127) // 128, K // 128))
    c = (rng.integers(-3000, 3000, (M, N)) * 0.0625).astype(np.float32)
    with _Cus(cus):
        D = _t(c)  # in place
        dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), D, D, _ws(dg.DG_OP_GEMM_NT, M, N, K))
        torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy(), oracle.gemm_nt_c(qa, sa, qb, sb, c))


# (cus, G, M, N, ks): 256 x 128 tiles without a cap, 256 x 256 tiles (the wide
# kernel) on capped CUs where the tiles of all groups fill whole rounds
KGROUPED = [(0, 3, 300, 160, [256, 0, 384]), (2, 3, 300, 272, [128, 384, 0]), (4, 2, 512, 512, [512, 256])]


@pytest.mark.parametrize("cus,G,M,N,ks", KGROUPED)
def test_k_grouped_varying_power_of_two_scales_bit_exact(cus, G, M, N, ks):
    rng = np.random.default_rng(G * 100 + M)
    ks = np.array(ks, np.int32)
    K = int(ks.sum())
    qa, qb = _codes(rng, M, K), _codes(rng, N, K)
    sa = _pow2(rng, (K // 128, M))
    sb = _pow2(rng, (K // 128, N))
    c = (rng.integers(-3000, 3000, (G, M, N)) * 0.0625).astype(np.float32)
    with _Cus(cus):
        D = _t(c)
        dg.dg_k_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, D, _t(ks))
        torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy(), oracle.k_grouped_contiguous(qa, sa, qb, sb, ks, c))


# (cus, counts, N, K): contiguous on 128 x 256 tiles, and on 256 x 256 tiles
# (tiles straddling two experts) on capped CUs, at a long and a short K
CONTIG = [(0, [130, 5, 256], 272, 512), (2, [200, 300, 40], 512, 4096), (2, [200, 300, 40], 512, 1024)]


@pytest.mark.parametrize("cus,counts,N,K", CONTIG)
def test_contiguous_varying_power_of_two_scales_bit_exact(cus, counts, N, K):
    rng = np.random.default_rng(sum(counts) + N)
    G = len(counts)
    padded = [(c + 127) // 128 * 128 for c in counts]
    m_total = sum(padded)
    idx = np.full(m_total, -1, np.int32)
    s = 0
    for e, (c, p) in enumerate(zip(counts, padded)):
        idx[s:s + c] = e
        s += p
    qa = _codes(rng, m_total, K)
    sa = _pow2(rng, (K // 128, m_total))
    qb = np.stack([_codes(rng, N, K) for _ in range(G)])
    sb = _pow2(rng, (G, (N + 127) // 128, K // 128))
    init = np.full((m_total, N), 0xFFFF, np.uint16)
    with _Cus(cus):
        D = _t(init.view(np.int16))
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(idx))
        torch.cuda.synchronize()
    got = D.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.grouped_contiguous(qa, sa, qb, sb, idx, init))


def test_masked_varying_power_of_two_scales_bit_exact():
    rng = np.random.default_rng(77)
    G, max_m, N, K = 5, 200, 400, 640
    mm = np.array([200, 0, 129, 1, 64], np.int32)
    qa = np.stack([_codes(rng, max_m, K) for _ in range(G)])
    sa = _pow2(rng, (G, K // 128, max_m))
    qb = np.stack([_codes(rng, N, K) for _ in range(G)])
    sb = _pow2(rng, (G, (N + 127) // 128, K // 128))
    init = np.full((G, max_m, N), 0xFFFF, np.uint16)
    D = _t(init.view(np.int16))
    dg.dg_m_grouped_fp8_gemm_nt_masked(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(mm))
    torch.cuda.synchronize()
    got = D.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.grouped_masked(qa, sa, qb, sb, mm, init))
