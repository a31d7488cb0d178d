"""The pins catch plausible mistakes: each test plants one mistake in a copy of
an oracle function (on the CPU) and checks that an independent pin rejects it."""

import numpy as np

from oracle import gemm as og
from oracle.bf16 import bf16_rne_bits
from oracle.e4m3 import decode_e4m3
from oracle.exact import gemm_nt_exact

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _case(M=2, N=200, K=384, seed=5):
    rng = np.random.default_rng(seed)
    a = FINITE[rng.integers(0, FINITE.size, (M, K))]
    b = FINITE[rng.integers(0, FINITE.size, (N, K))]
    sfa = rng.uniform(0.5, 2, (K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.5, 2, ((N + 127) // 128, K // 128)).astype(np.float32)
    return a, sfa, b, sfb


def _mutant(a_codes, sfa, b_codes, sfb, mistake):
    a = decode_e4m3(a_codes)
    b = decode_e4m3(b_codes)
    M, K = a.shape
    N = b.shape[0]
    if mistake == "b_transposed":  # B's bytes read as if stored [K, N]
        b = b.reshape(K, N).T
    nb = sfb.shape[0]
    acc = np.zeros((M, N))
    blocks = range(K // 128 - 1) if mistake == "drop_block" else range(K // 128)
    for g in blocks:
        ks = slice(128 * g, 128 * g + 128)
        p = a[:, ks] @ b[:, ks].T
        if mistake == "beta_mod":
            cb = np.arange(N) % nb
        else:
            cb = np.arange(N) // 128
        sa = sfa[g] if mistake != "alpha_wrong_group" else sfa[(g + 1) % (K // 128)]
        s = sa.astype(np.float64)[:, None] * sfb[cb, g].astype(np.float64)[None, :]
        if mistake == "sign":
            p = -p if g == 1 else p
        acc += s * p
    if mistake == "bf16_truncate":  # round toward zero through fp32 instead of RNE from fp64
        return (acc.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bf16_rne_bits(acc)


def _brute_force_rejects(mistake):
    a, sfa, b, sfb = _case()
    _, exact = gemm_nt_exact(a, sfa, b, sfb)
    assert np.array_equal(og.gemm_nt(a, sfa, b, sfb), exact)  # the real oracle passes
    return not np.array_equal(_mutant(a, sfa, b, sfb, mistake), exact)


def test_pin_rejects_wrong_beta_index():
    assert _brute_force_rejects("beta_mod")


def test_pin_rejects_dropped_k_block():
    assert _brute_force_rejects("drop_block")


def test_pin_rejects_wrong_alpha_group():
    assert _brute_force_rejects("alpha_wrong_group")


def test_pin_rejects_sign_error():
    assert _brute_force_rejects("sign")


def test_pin_rejects_transposed_operand():
    assert _brute_force_rejects("b_transposed")


def test_pin_rejects_truncating_epilogue():
    assert _brute_force_rejects("bf16_truncate")
