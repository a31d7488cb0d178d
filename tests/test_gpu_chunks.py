"""Calls the library splits into several launches, and operands past 4 GiB.

* Row chunks: a call whose rows exceed 32-bit byte offsets runs as row
  chunks launched back to back, each with its own plan (DG_FORCE_CONFIG=
  chunk_rows=<n> lowers the chunk size so small problems take that path: the
  last chunk may be a skinny one, contiguous segments may straddle chunk
  boundaries, and a split-K workspace is shared by the chunks).
* Many contiguous tiles per CU: the grid grows past a small CU cap so that
  no workgroup's tile table exceeds 64 entries.
* Real sizes past 4 GiB (sampled rows against the oracle): a dense A of
  4.3 GB (two chunks), and 40 experts of 7168 x 16384 weights (4.7 GB, every
  expert from its own base) in the masked and contiguous forms.
Every result is compared with the oracle (Lesson 13, Fig. 13-1 and Fig. 13-3):
bf16 outputs within 2^-7 |ref| + 1e-3 rms(ref), rows the operation does not
define bit-exact untouched."""

import os

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_matmul_amd import dg, workloads
from tests.helpers import SENTINEL, assert_close, assert_f32_rule

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _np16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class _Env:
    """Sets DG_FORCE_CONFIG (and DG_PRINT_CONFIGS) for the calls inside."""

    def __init__(self, force, cus=0):
        self.force = force
        self.cus = cus

    def __enter__(self):
        os.environ["DG_FORCE_CONFIG"] = self.force
        os.environ["DG_PRINT_CONFIGS"] = "1"
        dg.dg_set_num_cus(self.cus)

    def __exit__(self, *a):
        del os.environ["DG_FORCE_CONFIG"]
        del os.environ["DG_PRINT_CONFIGS"]
        dg.dg_set_num_cus(0)


def _launches(err, what):
    return [l for l in err.splitlines() if l.startswith(f"[dg] {what} ")]


def _dense_case(M, N, K, seed):
    a32, b32 = workloads.dense(M, N, K, seed)
    qa, sa = oracle.quant_1x128(a32)
    qb, sb = oracle.quant_128x128(b32)
    return qa, sa, qb, sb


def _ws(op, M, N, K):
    n = dg.dg_get_workspace_size(op, M, N, K, 1)
    return torch.zeros(max(n // 4, 1), dtype=torch.float32, device=DEV) if n else None


# (M, chunk_rows, kernel of the chunks): 600 rows in chunks of 256 end in an
# 88-row (skinny) chunk; 1000 rows in chunks of 512 on 256 x 256 tiles
DENSE = [(600, 256, ""), (700, 256, "kernel=persistent"), (1000, 512, "kernel=wide")]


@pytest.mark.parametrize("M,chunk,kernel", DENSE)
def test_dense_row_chunks(capfd, M, chunk, kernel):
    N, K = 400, 640
    qa, sa, qb, sb = _dense_case(M, N, K, seed=M)
    force = f"chunk_rows={chunk}" + (f",{kernel}" if kernel else "")
    D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
    capfd.readouterr()
    with _Env(force):
        dg.dg_fp8_gemm_nt(_t(qa), _t(sa), _t(qb), _t(sb), D, _ws(dg.DG_OP_GEMM_NT, M, N, K))
        torch.cuda.synchronize()
    launches = _launches(capfd.readouterr().err, "gemm_nt")
    assert len(launches) == -(-M // chunk), launches
    if M % chunk and M % chunk <= 128:
        assert "kernel=skinny" in launches[-1]
    assert_close(_np16(D), oracle.gemm_nt(qa, sa, qb, sb), f"dense {M} rows in chunks of {chunk}")


def test_acc_row_chunks_in_place(capfd):
    M, N, K = 600, 272, 512
    qa, sa, qb, sb = _dense_case(M, N, K, seed=3)
    c = (np.random.default_rng(4).standard_normal((M, N)) * 3).astype(np.float32)
    D = _t(c)
    capfd.readouterr()
    with _Env("chunk_rows=256"):
        dg.dg_fp8_gemm_nt_acc(_t(qa), _t(sa), _t(qb), _t(sb), D, D, _ws(dg.DG_OP_GEMM_NT, M, N, K))
        torch.cuda.synchronize()
    assert len(_launches(capfd.readouterr().err, "gemm_nt_acc")) == 3
    assert_f32_rule(D.cpu().numpy(), oracle.gemm_nt_c(qa, sa, qb, sb, c), "acc in row chunks")


def test_ue8m0_and_bf16_row_chunks(capfd):
    M, N, K = 700, 400, 640
    a32, b32 = workloads.dense(M, N, K, 5)
    qa, _, sa = oracle.quant_1x128_ue8m0(a32)
    qb, _, sb = oracle.quant_128x128_ue8m0(b32)
    D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
    a16, b16 = workloads.dense_bf16(M, N, K, 6)
    D2 = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
    capfd.readouterr()
    with _Env("chunk_rows=256"):
        dg.dg_fp8_gemm_nt_ue8m0(_t(qa), _t(sa), _t(qb), _t(sb), D, _ws(dg.DG_OP_GEMM_NT_UE8M0, M, N, K))
        dg.dg_bf16_gemm_nt(_t(a16.view(np.int16)), _t(b16.view(np.int16)), D2, _ws(dg.DG_OP_BF16_GEMM_NT, M, N, K))
        torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert len(_launches(err, "gemm_nt_ue8m0")) == 3 and len(_launches(err, "bf16_gemm_nt")) == 3
    assert_close(_np16(D), oracle.gemm_nt_ue8m0(qa, sa, qb, sb), "ue8m0 in row chunks")
    assert_close(_np16(D2), oracle.gemm_bf16_nt(a16, b16), "bf16 in row chunks")


def _contig(counts, N, K, seed):
    G = len(counts)
    w = workloads.contiguous(G, N, K, seed, counts=counts)
    qa, sa = oracle.quant_1x128(w["a"])
    qa, sa = workloads.place_rows(qa, sa, w["rows"], w["m_total"])
    qb, sb = oracle.quant_128x128(w["b"])
    return w, qa, sa, qb, sb


# segments of 300 / 130 rows straddle the 256-row chunk boundaries
@pytest.mark.parametrize("force", ["chunk_rows=256", "chunk_rows=256,kernel=wide", "chunk_rows=512,kernel=persistent"])
def test_contiguous_row_chunks(capfd, force):
    counts, N, K = [300, 5, 130, 1, 256, 77], 272, 512
    w, qa, sa, qb, sb = _contig(counts, N, K, seed=11)
    D = torch.full((w["m_total"], N), -1, dtype=torch.int16, device=DEV)
    capfd.readouterr()
    with _Env(force):
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(w["m_indices"]))
        torch.cuda.synchronize()
    chunk = int(force.split(",")[0].split("=")[1])
    launches = _launches(capfd.readouterr().err, "contiguous")
    assert len(launches) == -(-w["m_total"] // chunk)
    if "wide" in force:
        assert all("kernel=wide" in l for l in launches)
    got = _np16(D)
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, w["m_indices"], np.full(got.shape, SENTINEL, np.uint16))
    pad = w["m_indices"] < 0
    assert np.array_equal(got[pad], ref[pad])
    assert_close(got[~pad], ref[~pad], f"contiguous, {force}")


@pytest.mark.parametrize("kernel", ["persistent", "wide"])
def test_contiguous_more_than_64_tiles_per_cu(capfd, kernel):
    # one CU: 91 row blocks x 2 column tiles = 182 tiles of 128 x 256, or
    # 46 x 2 = 92 of 256 x 256 (the 128-row segments pair up in straddling
    # tiles); the grid grows to 3 or 2 workgroups
    counts = [130] * 40 + [5] * 11
    N, K = 512, 4096 if kernel == "wide" else 512
    w, qa, sa, qb, sb = _contig(counts, N, K, seed=21)
    D = torch.full((w["m_total"], N), -1, dtype=torch.int16, device=DEV)
    capfd.readouterr()
    with _Env(f"kernel={kernel}", cus=1):
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(_t(qa), _t(sa), _t(qb), _t(sb), D, _t(w["m_indices"]))
        torch.cuda.synchronize()
    (launch,) = _launches(capfd.readouterr().err, "contiguous")
    assert f"kernel={kernel}" in launch
    tiles = -(-w["m_total"] // (256 if kernel == "wide" else 128)) * 2
    assert tiles > 64 and f"grid={-(-tiles // 64)}" in launch
    got = _np16(D)
    ref = oracle.grouped_contiguous(qa, sa, qb, sb, w["m_indices"], np.full(got.shape, SENTINEL, np.uint16))
    pad = w["m_indices"] < 0
    assert np.array_equal(got[pad], ref[pad])
    assert_close(got[~pad], ref[~pad], f"contiguous {kernel} with many tiles on one CU")


# ---------------------------------------------------------------- past 4 GiB

def _random_codes(shape, gen):
    """Random finite e4m3 codes (0x00..0x7E, random sign) made on the device."""
    mag = torch.randint(0, 0x7F, shape, dtype=torch.uint8, device=DEV, generator=gen)
    sign = torch.randint(0, 2, shape, dtype=torch.uint8, device=DEV, generator=gen) << 7
    return mag | sign


def _scales(shape, gen):
    return torch.rand(shape, dtype=torch.float32, device=DEV, generator=gen) * 0.01 + 0.001


@pytest.mark.timeout(600)
def test_dense_activations_past_4_gib():
    # A of 262400 x 16384 bytes (4.3 GB): two row chunks, the first of 261632
    # rows (the most whose offsets fit 32 bits, rounded down to 256)
    M, N, K = 262400, 256, 16384
    assert "chunks=2" in dg.dg_describe_plan(dg.DG_OP_GEMM_NT, M, N, K)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    A = _random_codes((M, K), gen)
    SA = _scales((K // 128, M), gen)
    B = _random_codes((N, K), gen)
    SB = _scales((2, K // 128), gen)
    D = torch.full((M, N), -1, dtype=torch.int16, device=DEV)
    dg.dg_fp8_gemm_nt(A, SA, B, SB, D, _ws(dg.DG_OP_GEMM_NT, M, N, K))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 200000, 261631, 261632, 261633, M - 1])
    ri = torch.from_numpy(rows).to(DEV)
    qa = A.index_select(0, ri).cpu().numpy()
    sa = SA.index_select(1, ri).cpu().numpy()
    ref = oracle.gemm_nt(qa, sa, B.cpu().numpy(), SB.cpu().numpy())
    got = D.index_select(0, ri).cpu().numpy().view(np.uint16)
    del A
    assert_close(got, ref, "dense rows around the 4 GiB chunk boundary")


def _big_experts(G, N, K, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    B = _random_codes((G, N, K), gen)
    SB = _scales((G, (N + 127) // 128, K // 128), gen)
    return gen, B, SB


@pytest.mark.timeout(600)
def test_masked_weights_past_4_gib():
    # 40 experts of 7168 x 16384 (4.7 GB of weights; expert 36 straddles the
    # 4 GiB offset, experts 37 on start past it)
    G, max_m, N, K = 40, 8, 7168, 16384
    gen, B, SB = _big_experts(G, N, K, 8)
    A = _random_codes((G, max_m, K), gen)
    SA = _scales((G, K // 128, max_m), gen)
    mm = np.random.default_rng(9).integers(0, max_m + 1, G).astype(np.int32)
    mm[[0, 36, 38, 39]] = [max_m, 2, 3, 5]
    D = torch.full((G, max_m, N), -1, dtype=torch.int16, device=DEV)
    dg.dg_m_grouped_fp8_gemm_nt_masked(A, SA, B, SB, D, _t(mm))
    torch.cuda.synchronize()
    got = D.cpu().numpy().view(np.uint16)
    for g in (0, 21, 36, 38, 39):
        m = int(mm[g])
        ref = oracle.gemm_nt(A[g, :m].cpu().numpy(), SA[g, :, :m].cpu().numpy(), B[g].cpu().numpy(), SB[g].cpu().numpy())
        assert_close(got[g, :m], ref, f"masked expert {g}")
    for g in range(G):
        assert np.all(got[g, int(mm[g]):] == SENTINEL)


@pytest.mark.timeout(600)
def test_contiguous_weights_past_4_gib():
    G, N, K = 40, 7168, 16384
    gen, B, SB = _big_experts(G, N, K, 10)
    counts = np.random.default_rng(11).integers(1, 129, G)
    padded = (counts + 127) // 128 * 128
    m_total = int(padded.sum())
    idx = np.full(m_total, -1, np.int32)
    starts = np.concatenate([[0], np.cumsum(padded)[:-1]])
    for e in range(G):
        idx[starts[e]:starts[e] + counts[e]] = e
    A = _random_codes((m_total, K), gen)
    SA = _scales((K // 128, m_total), gen)
    D = torch.full((m_total, N), -1, dtype=torch.int16, device=DEV)
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(A, SA, B, SB, D, _t(idx))
    torch.cuda.synchronize()
    got = D.cpu().numpy().view(np.uint16)
    for e in (0, 20, 36, 39):
        rows = np.arange(starts[e], starts[e] + counts[e])
        ri = torch.from_numpy(rows).to(DEV)
        ref = oracle.gemm_nt(A.index_select(0, ri).cpu().numpy(), SA.index_select(1, ri).cpu().numpy(),
                             B[e].cpu().numpy(), SB[e].cpu().numpy())
        assert_close(got[rows], ref, f"contiguous expert {e}")
    assert np.all(got[idx < 0] == SENTINEL)
