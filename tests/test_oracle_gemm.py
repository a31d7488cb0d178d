"""Pins for the oracle GEMM (dense, contiguous, masked).

* exact rational brute force of the closed-form equation (Lesson 13, Fig. 13-1);
* integer exactness with unit scales;
* the page's worked exercise: promoted form vs dequantise-first form
  (tests/golden/lesson13_exercise.json);
* linearity in alpha and beta, and locality of each scale;
* grouped layouts reduce to per-expert dense results (Fig. 13-3).
"""

import json
import os

import numpy as np
import pytest

from oracle.bf16 import bf16_bits_to_f64, bf16_rne_bits
from oracle.e4m3 import decode_e4m3, encode_e4m3
from oracle.exact import gemm_nt_exact
from oracle.gemm import gemm_nt, gemm_nt_acc, grouped_contiguous, grouped_masked
from oracle.quant import quant_1x128, quant_128x128

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _rand_codes(rng, shape):
    return FINITE_CODES[rng.integers(0, FINITE_CODES.size, shape)]


def _rand_scales(rng, shape):
    return (rng.uniform(0.5, 2.0, shape) * np.exp2(rng.integers(-12, 4, shape))).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(2, 16, 128), (1, 136, 256), (2, 200, 384), (3, 16, 384)])
def test_brute_force_exact_rationals(M, N, K):
    rng = np.random.default_rng(M * 1000 + N + K)
    a = _rand_codes(rng, (M, K))
    b = _rand_codes(rng, (N, K))
    sfa = _rand_scales(rng, (K // 128, M))
    sfb = _rand_scales(rng, ((N + 127) // 128, K // 128))
    _, exact_bits = gemm_nt_exact(a, sfa, b, sfb)
    assert np.array_equal(gemm_nt(a, sfa, b, sfb), exact_bits)


def test_integer_exactness_unit_scales():
    rng = np.random.default_rng(11)
    M, N, K = 37, 200, 512
    ai = rng.integers(-10, 10, (M, K))
    bi = rng.integers(-10, 10, (N, K))
    a = encode_e4m3(ai.astype(np.float32))
    b = encode_e4m3(bi.astype(np.float32))
    assert np.array_equal(decode_e4m3(a), ai) and np.array_equal(decode_e4m3(b), bi)
    sfa = np.ones((K // 128, M), np.float32)
    sfb = np.ones(((N + 127) // 128, K // 128), np.float32)
    ref = ai.astype(np.int64) @ bi.astype(np.int64).T
    acc = gemm_nt_acc(a, sfa, b, sfb)
    assert np.array_equal(acc, ref.astype(np.float64))
    d = bf16_bits_to_f64(gemm_nt(a, sfa, b, sfb))
    small = np.abs(ref) <= 256
    assert np.array_equal(d[small], ref[small].astype(np.float64))


def test_pages_worked_exercise_promoted_equals_dequantise_first():
    g = json.load(open(os.path.join(GOLDEN, "lesson13_exercise.json")))
    M, N, K, bk, bn = g["M"], g["N"], g["K"], g["block_k"], g["block_n"]
    rs = np.random.RandomState(g["seed"])
    A = rs.randint(g["int_low"], g["int_high_exclusive"], size=(M, K)).astype(np.float32)
    B = rs.randint(g["int_low"], g["int_high_exclusive"], size=(N, K)).astype(np.float32)
    S_A = rs.uniform(g["scale_low"], g["scale_high"], size=(M, K // bk)).astype(np.float32)
    S_B = rs.uniform(g["scale_low"], g["scale_high"], size=(N // bn, K // bk)).astype(np.float32)
    # the dequantise-first reading of the closed form: expand every scale to
    # the elements it covers (alpha over its row's 128-wide K group, beta over
    # its 128 x 128 block), dequantise both operands once, and take one
    # ordinary product of the real-valued matrices
    alpha_full = np.repeat(S_A.astype(np.float64), bk, axis=1)                  # [M, K]
    beta_full = np.repeat(np.repeat(S_B.astype(np.float64), bn, axis=0), bk, axis=1)  # [N, K]
    a_real = A.astype(np.float64) * alpha_full
    b_real = B.astype(np.float64) * beta_full
    deq = a_real @ b_real.T
    acc = gemm_nt_acc(encode_e4m3(A), np.ascontiguousarray(S_A.T), encode_e4m3(B), S_B)
    assert np.allclose(acc, deq, atol=g["atol"], rtol=0)
    # both are fp64 evaluations of the same sum: they differ by rounding only,
    # bounded by a few ulps of the sum of the absolute terms
    mag = np.abs(a_real) @ np.abs(b_real).T
    assert np.all(np.abs(acc - deq) <= 4 * (K // bk + 1) * 2.0 ** -53 * mag * 8)


def test_linearity_power_of_two_bit_exact_and_locality():
    rng = np.random.default_rng(12)
    M, N, K = 9, 264, 384
    a = _rand_codes(rng, (M, K))
    b = _rand_codes(rng, (N, K))
    sfa = _rand_scales(rng, (K // 128, M))
    sfb = _rand_scales(rng, ((N + 127) // 128, K // 128))
    base = gemm_nt_acc(a, sfa, b, sfb)
    # alpha -> 4 alpha for every group scales D by 4 exactly
    assert np.array_equal(gemm_nt_acc(a, sfa * np.float32(4), b, sfb), base * 4)
    assert np.array_equal(gemm_nt_acc(a, sfa, b, sfb * np.float32(0.125)), base * 0.125)
    bits = gemm_nt(a, sfa, b, sfb)
    assert np.array_equal(bf16_bits_to_f64(gemm_nt(a, sfa * np.float32(2), b, sfb)), bf16_bits_to_f64(bits) * 2)
    # changing alpha[g, i] changes only row i
    s2 = sfa.copy()
    s2[1, 4] *= np.float32(1.7)
    d = gemm_nt_acc(a, s2, b, sfb) != base
    assert d[4].any() and not np.delete(d, 4, axis=0).any()
    # changing beta[nb, g] changes only the columns of block nb
    t2 = sfb.copy()
    t2[1, 2] *= np.float32(0.3)
    d = gemm_nt_acc(a, sfa, b, t2) != base
    assert d[:, 128:256].any() and not d[:, :128].any() and not d[:, 256:].any()
    # general factor: linear within fp64 rounding
    c = np.float32(1.37)
    mag = gemm_nt_acc(a & 0x7F, sfa, b & 0x7F, sfb)  # sum of |terms|
    assert np.all(np.abs(gemm_nt_acc(a, sfa * c, b, sfb) - base * np.float64(c)) <= 1e-6 * mag)


def test_quantised_gemm_approximates_fp32_product():
    # end-to-end sanity: quantise fp32 sources, GEMM, compare with the fp64 product
    rng = np.random.default_rng(13)
    x = rng.standard_normal((64, 1024), dtype=np.float32)
    w = rng.standard_normal((136, 1024), dtype=np.float32) / np.float32(32)
    qa, sa = quant_1x128(x)
    qb, sb = quant_128x128(w)
    d = bf16_bits_to_f64(gemm_nt(qa, sa, qb, sb))
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(d - ref) / np.linalg.norm(ref)
    assert rel < 0.05


def _grouped_case(rng, G, N, K, counts):
    pad = (counts + 127) // 128 * 128
    m_total = int(pad.sum())
    m_idx = np.full(m_total, -1, np.int32)
    s = 0
    for e in range(G):
        m_idx[s:s + counts[e]] = e
        s += pad[e]
    a = _rand_codes(rng, (m_total, K))
    sfa = _rand_scales(rng, (K // 128, m_total))
    b = _rand_codes(rng, (G, N, K))
    sfb = _rand_scales(rng, (G, (N + 127) // 128, K // 128))
    return m_idx, a, sfa, b, sfb


def test_contiguous_equals_per_expert_dense_and_leaves_padding():
    rng = np.random.default_rng(14)
    G, N, K = 3, 144, 256
    counts = np.array([5, 130, 1])
    m_idx, a, sfa, b, sfb = _grouped_case(rng, G, N, K, counts)
    d0 = np.full((m_idx.size, N), 0xFFFF, np.uint16)
    d = grouped_contiguous(a, sfa, b, sfb, m_idx, d0)
    for i in range(m_idx.size):
        e = m_idx[i]
        if e < 0:
            assert np.all(d[i] == 0xFFFF)
        else:
            assert np.array_equal(d[i], gemm_nt(a[i:i + 1], sfa[:, i:i + 1], b[e], sfb[e])[0])


def test_contiguous_single_group_equals_dense_and_permutation():
    rng = np.random.default_rng(15)
    N, K = 128, 256
    a = _rand_codes(rng, (256, K))
    sfa = _rand_scales(rng, (2, 256))
    b = _rand_codes(rng, (2, N, K))
    sfb = _rand_scales(rng, (2, 1, 2))
    m_idx = np.zeros(256, np.int32)
    d0 = np.zeros((256, N), np.uint16)
    assert np.array_equal(grouped_contiguous(a, sfa, b[:1], sfb[:1], m_idx, d0), gemm_nt(a, sfa, b[0], sfb[0]))
    # two segments of 128 rows; swapping the segments (rows and tags) swaps the outputs
    m_idx = np.repeat(np.array([0, 1], np.int32), 128)
    d = grouped_contiguous(a, sfa, b, sfb, m_idx, d0)
    perm = np.concatenate([np.arange(128, 256), np.arange(128)])
    d2 = grouped_contiguous(a[perm], sfa[:, perm], b, sfb, m_idx[perm], d0)
    assert np.array_equal(d2, d[perm])


def test_out_of_range_indices_are_padding():
    rng = np.random.default_rng(16)
    m_idx, a, sfa, b, sfb = _grouped_case(rng, 2, 16, 128, np.array([3, 4]))
    m_idx2 = m_idx.copy()
    m_idx2[0] = 2  # == G: out of range
    m_idx2[1] = -7
    d0 = np.full((m_idx.size, 16), 0x1234, np.uint16)
    d = grouped_contiguous(a, sfa, b, sfb, m_idx2, d0)
    assert np.all(d[0] == 0x1234) and np.all(d[1] == 0x1234)
    assert np.array_equal(d[2:], grouped_contiguous(a, sfa, b, sfb, m_idx, d0)[2:])


def test_masked_equals_dense_and_clamps():
    rng = np.random.default_rng(17)
    G, max_m, N, K = 4, 8, 136, 256
    a = _rand_codes(rng, (G, max_m, K))
    sfa = _rand_scales(rng, (G, K // 128, max_m))
    b = _rand_codes(rng, (G, N, K))
    sfb = _rand_scales(rng, (G, 2, K // 128))
    d0 = np.full((G, max_m, N), 0xFFFF, np.uint16)
    mm = np.array([max_m, 0, 3, 99], np.int32)  # full, empty, partial, clamped
    d = grouped_masked(a, sfa, b, sfb, mm, d0)
    assert np.array_equal(d[0], gemm_nt(a[0], sfa[0], b[0], sfb[0]))
    assert np.all(d[1] == 0xFFFF)
    assert np.array_equal(d[2, :3], gemm_nt(a[2, :3], sfa[2][:, :3], b[2], sfb[2]))
    assert np.all(d[2, 3:] == 0xFFFF)
    assert np.array_equal(d[3], gemm_nt(a[3], sfa[3], b[3], sfb[3]))
    d_neg = grouped_masked(a, sfa, b, sfb, np.array([-1, -5, 0, 0], np.int32), d0)
    assert np.all(d_neg == 0xFFFF)


def test_nan_codes_only_reach_their_own_rows():
    # trap bytes in one row of A poison only that row (the GEMM never mixes rows)
    rng = np.random.default_rng(18)
    a = _rand_codes(rng, (4, 128))
    a[2, 7] = 0x7F
    b = _rand_codes(rng, (16, 128))
    d = bf16_bits_to_f64(gemm_nt(a, np.ones((1, 4), np.float32), b, np.ones((1, 1), np.float32)))
    assert np.all(np.isnan(d[2])) and not np.isnan(np.delete(d, 2, axis=0)).any()
