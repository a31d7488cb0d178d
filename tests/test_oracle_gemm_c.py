"""Pins of the accumulating FP8 GEMM oracle (oracle.gemm_nt_c, D = C + A.B^T
in fp32) to things other than itself: exact rational brute force, numpy's
independent fp64 -> fp32 cast for the rounding helper, integer exactness and
planted mistakes."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm_nt_acc, gemm_nt_c
from oracle.exact import f32_from_fraction, gemm_nt_c_exact

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _case(M, N, K, seed, c_scale=1.0):
    rng = np.random.default_rng(seed)
    a = FINITE[rng.integers(0, FINITE.size, (M, K))]
    b = FINITE[rng.integers(0, FINITE.size, (N, K))]
    sfa = rng.uniform(0.5, 2, (K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.5, 2, ((N + 127) // 128, K // 128)).astype(np.float32)
    acc = gemm_nt_acc(a, sfa, b, sfb)
    # C of the product's size and of opposite sign where it cancels most
    c = (-acc * rng.uniform(0.9, 1.1, acc.shape) * c_scale).astype(np.float32)
    return a, sfa, b, sfb, c


def test_f32_rounding_helper_matches_numpy():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000))
    for v in x:
        assert f32_from_fraction(Fraction(float(v))) == np.float32(v) or (np.isinf(np.float32(v)))


@pytest.mark.parametrize("M,N,K,seed,c_scale", [(2, 3, 128, 1, 1.0), (3, 2, 256, 2, 0.0), (2, 2, 128, 3, 1e-3)])
def test_gemm_c_equals_exact_rational(M, N, K, seed, c_scale):
    a, sfa, b, sfb, c = _case(M, N, K, seed, c_scale)
    got = gemm_nt_c(a, sfa, b, sfb, c)
    ref = gemm_nt_c_exact(a, sfa, b, sfb, c)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_gemm_c_integer_inputs_exact():
    from oracle import encode_e4m3
    rng = np.random.default_rng(4)
    M, N, K = 5, 7, 256
    qa = encode_e4m3(rng.integers(-10, 10, (M, K)).astype(np.float32))
    qb = encode_e4m3(rng.integers(-10, 10, (N, K)).astype(np.float32))
    c = rng.integers(-1000, 1000, (M, N)).astype(np.float32)
    ones_a = np.ones((K // 128, M), np.float32)
    ones_b = np.ones(((N + 127) // 128, K // 128), np.float32)
    from oracle import decode_e4m3
    ref = decode_e4m3(qa) @ decode_e4m3(qb).T + c
    assert np.array_equal(gemm_nt_c(qa, ones_a, qb, ones_b, c), ref.astype(np.float32))


def test_gemm_c_none_is_zero():
    a, sfa, b, sfb, _ = _case(4, 130, 256, 5)
    z = np.zeros((4, 130), np.float32)
    assert np.array_equal(gemm_nt_c(a, sfa, b, sfb, None), gemm_nt_c(a, sfa, b, sfb, z))


@pytest.mark.parametrize("mistake", ["c_twice", "c_dropped", "round_twice"])
def test_planted_mistakes_fail_the_exact_pin(mistake):
    a, sfa, b, sfb, c = _case(2, 3, 256, 6, 1.0)
    acc = gemm_nt_acc(a, sfa, b, sfb)
    if mistake == "c_twice":
        bad = (acc + 2 * c.astype(np.float64)).astype(np.float32)
    elif mistake == "c_dropped":
        bad = acc.astype(np.float32)
    else:  # accumulator rounded to fp32 before C is added
        bad = (acc.astype(np.float32) + c).astype(np.float32)
    ref = gemm_nt_c_exact(a, sfa, b, sfb, c)
    assert not np.array_equal(bad.view(np.uint32), ref.view(np.uint32))
