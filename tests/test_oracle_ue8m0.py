"""Pins of the UE8M0 oracle (oracle/ue8m0.py) to things other than itself:
the code's defining inequality checked with exact integer arithmetic, exact
powers of two as closed forms, torch's independent float8 cast for the
quantised bytes, an explicit byte layout for the packing, exact rational
brute force for the GEMM, and planted mistakes (a scale rounded down, the
packing's byte order reversed)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import decode_e4m3, gemm_nt_ue8m0, quant_128x128_ue8m0, quant_1x128_ue8m0
from oracle.exact import gemm_nt_exact
from oracle.ue8m0 import pack_k, ue8m0_code, ue8m0_value, unpack_k


def _amax_samples():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4000) * np.exp2(rng.integers(-140, 120, 4000))).astype(np.float32)
    edges = []
    for k in range(-120, 110, 7):
        p = np.float32(448.0 * 2.0 ** k)
        edges += [p, np.nextafter(p, np.float32(np.inf)), np.nextafter(p, np.float32(0))]
    tiny = [np.float32(1e-45), np.float32(2.0 ** -126), np.float32(448.0 * 2.0 ** -128)]
    return np.abs(np.concatenate([x, np.array(edges + tiny, np.float32)]))


def test_code_is_smallest_power_of_two_not_below_amax_over_448():
    amax = _amax_samples()
    codes = ue8m0_code(amax)
    for a, c in zip(amax, codes):
        fa = Fraction(float(a))
        e = int(c) - 127
        if a == 0:
            assert c == 127
            continue
        if c > 0:  # unclamped: 448 * 2^(e-1) < amax <= 448 * 2^e
            assert 448 * Fraction(2) ** e >= fa
            assert 448 * Fraction(2) ** (e - 1) < fa
        else:  # clamped at 2^-127: still no saturation
            assert 448 * Fraction(2) ** -127 >= fa


def test_codes_of_exact_powers():
    for k in range(-100, 100, 3):
        assert ue8m0_code(np.float32(448.0 * 2.0 ** k)) == 127 + k
        assert ue8m0_code(np.nextafter(np.float32(448.0 * 2.0 ** k), np.float32(np.inf))) == 128 + k
    assert ue8m0_code(np.float32(0.0)) == 127
    assert ue8m0_value(np.array([0, 127, 254])).tolist() == [2.0 ** -127, 1.0, 2.0 ** 127]


def test_quantised_bytes_match_torch_float8_cast():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 512)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    x[3, :128] = 0.0
    x[5, 130] = 1e-30
    q, codes, packed = quant_1x128_ue8m0(x)
    scale = ue8m0_value(codes).T  # [M, kb]
    y = torch.from_numpy(x.reshape(64, 4, 128).astype(np.float64) / scale[..., None].astype(np.float64))
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(64, 512)
    assert np.array_equal(q, ref)
    assert np.all(np.abs(decode_e4m3(q)) <= 448)
    # no saturation, and the group maximum (in (224, 448] before rounding) stays in the top binade
    g = np.abs(decode_e4m3(q)).reshape(64, 4, 128).max(axis=2)
    assert np.all((g >= 224) | (g == 0) | (codes.T == 0))


def test_weight_blocks_and_ragged_rows():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 256)).astype(np.float32)
    q, codes, packed = quant_128x128_ue8m0(x)
    assert codes.shape == (2, 2) and packed.shape == (2, 1)
    for b in range(2):
        r0, r1 = 128 * b, min(128 * b + 128, 200)
        for k in range(2):
            amax = np.abs(x[r0:r1, 128 * k:128 * k + 128]).max()
            assert codes[b, k] == ue8m0_code(amax)


def test_packing_byte_layout():
    codes = np.array([[1, 2, 3, 4, 5]], np.uint8)
    words = pack_k(codes).view(np.uint32)
    assert words.tolist() == [[0x04030201, 0x00000005]]
    assert np.array_equal(unpack_k(pack_k(codes), 5), codes)


def test_ue8m0_gemm_equals_exact_rational():
    rng = np.random.default_rng(3)
    a32 = rng.standard_normal((3, 256)).astype(np.float32) * 5
    b32 = rng.standard_normal((4, 256)).astype(np.float32) / 16
    qa, ca, pa = quant_1x128_ue8m0(a32)
    qb, cb, pb = quant_128x128_ue8m0(b32)
    got = gemm_nt_ue8m0(qa, pa, qb, pb)
    _, ref = gemm_nt_exact(qa, ue8m0_value(ca), qb, ue8m0_value(cb))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("mistake", ["round_down", "byte_order"])
def test_planted_mistakes_are_caught(mistake):
    if mistake == "round_down":
        # floor instead of ceil: some group then needs values above 448
        amax = _amax_samples()
        amax = amax[amax > 1e-30]
        bad = (127 + np.floor(np.log2(amax.astype(np.float64) / 448.0))).astype(np.int64)
        over = amax.astype(np.float64) / np.ldexp(1.0, bad - 127) > 448
        assert over.any() and not np.array_equal(bad, ue8m0_code(amax))
    else:
        c = np.array([[1, 2, 3, 4]], np.uint8)
        rev = (c[:, 3].astype(np.uint32) | (c[:, 2].astype(np.uint32) << 8) | (c[:, 1].astype(np.uint32) << 16)
               | (c[:, 0].astype(np.uint32) << 24))
        assert rev[0] != pack_k(c).view(np.uint32)[0, 0]


# ---- grouped forms with UE8M0 scales: every computed row equals the exact
# rational GEMM of its expert (decoded powers of two), every other row keeps
# its prior contents; a planted mistake (the first expert's weight codes used
# for every expert) is caught

def _grouped_case(rng, G, N, K):
    from oracle.ue8m0 import quant_128x128_ue8m0 as qw

    b = [qw((rng.standard_normal((N, K)) / 8 * 2.0 ** rng.integers(-3, 4)).astype(np.float32)) for _ in range(G)]
    qb = np.stack([x[0] for x in b])
    cb = np.stack([x[1] for x in b])
    pb = np.stack([x[2] for x in b])
    return qb, cb, pb


def test_grouped_contiguous_ue8m0_equals_exact_rational_per_expert():
    from oracle import grouped_contiguous_ue8m0

    rng = np.random.default_rng(21)
    G, N, K = 3, 16, 640
    counts = [2, 0, 3]
    idx = np.array([0, 0, -1, 2, 2, 2, 7], np.int32)  # -1 and 7: untouched
    a32 = (rng.standard_normal((len(idx), K)) * 2.0 ** rng.integers(-4, 5, (len(idx), 1))).astype(np.float32)
    qa, ca, pa = quant_1x128_ue8m0(a32)
    qb, cb, pb = _grouped_case(rng, G, N, K)
    init = rng.integers(0, 1 << 16, (len(idx), N)).astype(np.uint16)
    got = grouped_contiguous_ue8m0(qa, pa, qb, pb, idx, init)
    for r, e in enumerate(idx):
        if 0 <= e < G:
            _, ref = gemm_nt_exact(qa[r:r + 1], ue8m0_value(ca[:, r:r + 1]), qb[e], ue8m0_value(cb[e]))
            assert np.array_equal(got[r:r + 1], ref), r
        else:
            assert np.array_equal(got[r], init[r])
    assert sum(counts) == int(np.sum((idx >= 0) & (idx < G)))
    # planted mistake: expert 0's weight codes for every expert
    wrong = grouped_contiguous_ue8m0(qa, pa, qb, np.broadcast_to(pb[:1], pb.shape), idx, init)
    assert not np.array_equal(wrong, got)


def test_grouped_masked_ue8m0_equals_exact_rational_per_expert():
    from oracle import grouped_masked_ue8m0

    rng = np.random.default_rng(22)
    G, max_m, N, K = 3, 4, 16, 512
    mm = np.array([4, -2, 9], np.int32)  # clamped to 4, 0, 4
    a32 = (rng.standard_normal((G * max_m, K)) * 2.0 ** rng.integers(-4, 5, (G * max_m, 1))).astype(np.float32)
    qa, ca, pa = quant_1x128_ue8m0(a32)
    qa = qa.reshape(G, max_m, K)
    ca = np.ascontiguousarray(ca.reshape(K // 128, G, max_m).transpose(1, 0, 2))
    pa = np.ascontiguousarray(pa.reshape(pa.shape[0], G, max_m).transpose(1, 0, 2))
    qb, cb, pb = _grouped_case(rng, G, N, K)
    init = rng.integers(0, 1 << 16, (G, max_m, N)).astype(np.uint16)
    got = grouped_masked_ue8m0(qa, pa, qb, pb, mm, init)
    for g in range(G):
        m = min(max(int(mm[g]), 0), max_m)
        if m:
            _, ref = gemm_nt_exact(qa[g, :m], ue8m0_value(ca[g][:, :m]), qb[g], ue8m0_value(cb[g]))
            assert np.array_equal(got[g, :m], ref)
        assert np.array_equal(got[g, m:], init[g, m:])
    wrong = grouped_masked_ue8m0(qa, pa, qb, np.broadcast_to(pb[:1], pb.shape), mm, init)
    assert not np.array_equal(wrong, got)
