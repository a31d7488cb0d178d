"""Pins for the oracle's number formats: e4m3 decode/encode and bf16 rounding.

Each is checked against something other than itself: torch's independent
float8_e4m3fn / bfloat16 casts, exact rational rounding, and the format facts
the pages print (tests/golden/e4m3_format.json).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.e4m3 import DECODE_TABLE, E4M3_MAX, decode_e4m3, encode_e4m3
from oracle.bf16 import bf16_bits_to_f64, bf16_rne_bits
from oracle.exact import bf16_bits_from_fraction, e4m3_fraction

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_decode():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_facts_from_pages():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_format.json")))
    finite = DECODE_TABLE[np.isfinite(DECODE_TABLE)]
    assert finite.max() == g["max_finite"] == E4M3_MAX
    assert finite.min() == -g["max_finite"]
    # 4 exponent + 3 mantissa bits: 2^4 binades of 2^3 steps, minus one NaN pattern per sign
    assert np.isnan(DECODE_TABLE).sum() == 2
    assert np.unique(finite).size == 2 ** (1 + g["exponent_bits"] + g["mantissa_bits"]) - 2 - 1  # +-0 merge


def test_e4m3_decode_matches_torch_all_codes():
    ours = decode_e4m3(np.arange(256))
    ref = _torch_e4m3_decode()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_e4m3_decode_matches_exact_fractions():
    for c in range(256):
        f = e4m3_fraction(c)
        if f is None:
            assert np.isnan(DECODE_TABLE[c])
        else:
            assert Fraction(DECODE_TABLE[c]) == f


def test_e4m3_special_values():
    assert DECODE_TABLE[0x01] == 2.0 ** -9  # smallest subnormal
    assert DECODE_TABLE[0x08] == 2.0 ** -6  # smallest normal
    assert DECODE_TABLE[0x38] == 1.0
    assert DECODE_TABLE[0x7E] == 448.0
    # every integer up to 16 is exact, above that only even ones up to 32
    vals = set(DECODE_TABLE[np.isfinite(DECODE_TABLE)].tolist())
    assert all(float(i) in vals for i in range(17))
    assert 17.0 not in vals and 18.0 in vals


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes)), codes)


def test_e4m3_encode_matches_torch_dense_fp32_sweep():
    # every 5th fp32 bit pattern from 2^-12 up to 448, both signs (~22M values)
    lo = np.float32(2.0 ** -12).view(np.uint32)
    hi = np.float32(448.0).view(np.uint32)
    for start in range(int(lo), int(hi) + 1, 5 * 2 ** 20):
        bits = np.arange(start, min(start + 5 * 2 ** 20, int(hi) + 1), 5, dtype=np.uint32)
        x = bits.view(np.float32)
        x = np.concatenate([x, -x])
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(encode_e4m3(x), ref)


def test_e4m3_encode_ties_go_to_even():
    finite = np.sort(np.unique(DECODE_TABLE[(DECODE_TABLE >= 0) & np.isfinite(DECODE_TABLE)]))
    mids = (finite[:-1] + finite[1:]) / 2  # exact in fp64 and fp32
    codes = encode_e4m3(mids.astype(np.float32))
    assert np.all(codes & 1 == 0)
    # and each tie lands on one of its two neighbours
    dec = decode_e4m3(codes)
    assert np.all((dec == finite[:-1]) | (dec == finite[1:]))
    ref = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_e4m3_sign_and_saturation_conventions():
    assert encode_e4m3(np.float32(-1e-4)) == 0x80  # sign-preserving zero
    assert encode_e4m3(np.float32(0.0)) == 0x00
    assert encode_e4m3(np.float32(-0.0)) == 0x80
    assert encode_e4m3(np.float32(448.0)) == 0x7E
    assert encode_e4m3(np.float32(448.00003)) == 0x7E
    assert encode_e4m3(np.float32(1000.0)) == 0x7E
    assert encode_e4m3(np.float32(-1000.0)) == 0xFE
    assert encode_e4m3(np.float32(np.nan)) & 0x7F == 0x7F


def test_bf16_matches_torch_for_fp32_inputs():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16_rne_bits(x.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_matches_exact_rational_rounding():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000))
    # constructed ties and near-ties in fp64 that fp32 cannot hold
    base = np.float64(1.0 + 2.0 ** -8)
    extra = np.array([base, base + 2.0 ** -40, base - 2.0 ** -40, 1 + 3 * 2.0 ** -8, -(1 + 3 * 2.0 ** -8),
                      2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, (2 - 2.0 ** -8) * 2.0 ** 127])
    for v in np.concatenate([x, extra]):
        assert int(bf16_rne_bits(v)) == bf16_bits_from_fraction(Fraction(float(v))), v


def test_bf16_rounds_once_from_fp64():
    # 1 + 2^-8 + 2^-30 is above the tie between 1 and 1 + 2^-7; rounding through
    # fp32 first would land exactly on the tie and then go to 1.0
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert bf16_bits_to_f64(bf16_rne_bits(v)) == 1.0 + 2.0 ** -7
    assert bf16_bits_to_f64(bf16_rne_bits(np.float64(np.float32(v)))) == 1.0


def test_bf16_specials():
    assert int(bf16_rne_bits(-0.0)) == 0x8000
    assert int(bf16_rne_bits(1e300)) == 0x7F80
    assert int(bf16_rne_bits(-1e300)) == 0xFF80
    assert np.isnan(bf16_bits_to_f64(bf16_rne_bits(np.nan)))
    assert bf16_bits_to_f64(bf16_rne_bits(3.0)) == 3.0
