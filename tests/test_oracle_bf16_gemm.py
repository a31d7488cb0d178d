"""Pins of the BF16 GEMM oracle (oracle/gemm_bf16.py) to things other than
itself: torch's bfloat16 cast for the decoding, exact rational brute force
for the sum and the rounding, integer exactness, and planted mistakes that a
pin must reject."""

import numpy as np
import pytest
import torch

from oracle.bf16 import bf16_bits_to_f64, bf16_rne_bits
from oracle.exact import bf16_fraction, gemm_bf16_nt_exact
from oracle.gemm_bf16 import gemm_bf16_nt


def test_bf16_decode_matches_torch_for_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # the NaN patterns
        ours = bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    for c in (0x0001, 0x3F80, 0xC0A0, 0x7F7F, 0x0080):  # subnormal, 1, -5, max, min normal
        assert float(bf16_fraction(c)) == ours[c]


def _random_bits(rng, shape, lo=-20, hi=20):
    x = rng.standard_normal(shape) * np.exp2(rng.integers(lo, hi, shape))
    return bf16_rne_bits(x)


@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 64, 0), (2, 7, 128, 1), (4, 3, 192, 2)])
def test_bf16_gemm_equals_exact_rational(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = _random_bits(rng, (M, K))
    b = _random_bits(rng, (N, K))
    assert np.array_equal(gemm_bf16_nt(a, b), gemm_bf16_nt_exact(a, b))


def test_bf16_gemm_integer_inputs_exact():
    # integers in [-3, 3] with K = 16: every dot product is an integer of
    # magnitude <= 144, exactly representable in bf16 (8 significant bits)
    rng = np.random.default_rng(7)
    a_int = rng.integers(-3, 4, (9, 16))
    b_int = rng.integers(-3, 4, (11, 16))
    got = bf16_bits_to_f64(gemm_bf16_nt(bf16_rne_bits(a_int), bf16_rne_bits(b_int)))
    assert np.array_equal(got, (a_int @ b_int.T).astype(np.float64))


def _mutant(a_bits, b_bits, mistake):
    a = bf16_bits_to_f64(a_bits)
    b = bf16_bits_to_f64(b_bits)
    K = a.shape[1]
    if mistake == "b_transposed":  # B's bytes read as if stored [K, N]
        b = b.reshape(K, -1).T
    if mistake == "drop_chunk":  # the last 64-wide K chunk left out
        a, b = a[:, :K - 64], b[:, :K - 64]
    if mistake == "fp32_sum":  # products summed in fp32 and rounded twice
        return bf16_rne_bits((a.astype(np.float32) @ b.astype(np.float32).T).astype(np.float64))
    return bf16_rne_bits(a @ b.T)


@pytest.mark.parametrize("mistake", ["b_transposed", "drop_chunk"])
def test_planted_mistakes_fail_the_exact_pin(mistake):
    rng = np.random.default_rng(3)
    M, N, K = 3, 128, 128  # square-able shapes so the transposed read is well formed
    a = _random_bits(rng, (M, K), -4, 4)
    b = _random_bits(rng, (N, K), -4, 4)
    exact = gemm_bf16_nt_exact(a, b)
    assert np.array_equal(_mutant(a, b, "none"), exact)
    assert not np.array_equal(_mutant(a, b, mistake), exact)
