"""Pins for the oracle quantisers (1x128 activation groups, 128x128 weight blocks).

The rule comes from Lesson 13, Fig. 13-1: scale = group amax / 448.  Checked
against an independent composition in torch, invariants of the rule and the
stored layouts.
"""

import json
import os

import numpy as np
import torch

from oracle.e4m3 import decode_e4m3
from oracle.quant import quant_1x128, quant_128x128

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _src(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    m = rng.random(shape, dtype=np.float32) < 1e-3
    x[m] *= 20
    return x * np.exp2(rng.integers(-20, 20, shape[:-1] + (1,))).astype(np.float32)


def _torch_1x128(x):
    t = torch.from_numpy(x)
    M, K = t.shape
    g = t.view(M, K // 128, 128)
    amax = g.abs().amax(dim=2)
    alpha = amax / torch.tensor(448.0, dtype=torch.float32)
    alpha = torch.where(alpha == 0, torch.ones_like(alpha), alpha)
    q = (g / alpha[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(M, K)
    return q.numpy(), alpha.T.contiguous().numpy()


def test_scale_divisor_is_the_pages_e4m3_max():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_format.json")))
    x = np.zeros((1, 128), np.float32)
    x[0, 5] = 7.0
    _, s = quant_1x128(x)
    assert s[0, 0] == np.float32(7.0) / np.float32(g["scale_divisor"])


def test_1x128_matches_independent_torch_composition():
    x = _src((96, 1024), 3)
    q, s = quant_1x128(x)
    qt, st = _torch_1x128(x)
    assert s.shape == (1024 // 128, 96)
    assert np.array_equal(s.view(np.uint32), st.view(np.uint32))
    assert np.array_equal(q, qt)


def test_1x128_amax_element_encodes_to_448():
    x = _src((300, 512), 4)
    q, _ = quant_1x128(x)
    g = x.reshape(300, 4, 128)
    idx = np.abs(g).argmax(axis=2)
    qa = q.reshape(300, 4, 128)
    picked = np.take_along_axis(qa, idx[..., None], axis=2)[..., 0]
    assert np.all((picked & 0x7F) == 0x7E)


def test_1x128_error_bound():
    x = _src((64, 384), 5)
    q, s = quant_1x128(x)
    deq = decode_e4m3(q).reshape(64, 3, 128) * s.T[..., None].astype(np.float64)
    err = np.abs(deq - x.reshape(64, 3, 128))
    # half an e4m3 ulp of the scaled value, ulp = 2^(floor(log2|y|) - 3), at least 2^-9
    y = np.abs(x.reshape(64, 3, 128) / s.T[..., None])
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.maximum(y, 1e-30))), -6) - 3)
    assert np.all(err <= 0.5 * ulp * s.T[..., None] * (1 + 1e-6) + 1e-30)


def test_1x128_power_of_two_rescale():
    x = _src((32, 256), 6)
    q, s = quant_1x128(x)
    for sh in (-5, 3, 17):
        q2, s2 = quant_1x128(x * np.float32(2.0 ** sh))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** sh))


def test_1x128_zero_group_convention():
    # parity unpinned: no page fixes the all-zero group; convention alpha = 1, codes +-0
    x = np.zeros((2, 256), np.float32)
    x[0, :128] = -0.0
    x[1, 128:] = np.linspace(-1, 1, 128)
    q, s = quant_1x128(x)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert np.all(q[0, :128] == 0x80) and np.all(q[0, 128:] == 0)
    assert s[1, 1] == np.float32(1.0) / np.float32(448.0)


def test_1x128_grouped_layout():
    x = _src((3, 40, 256), 7)
    q, s = quant_1x128(x)
    assert q.shape == (3, 40, 256) and s.shape == (3, 2, 40)
    for g in range(3):
        q1, s1 = quant_1x128(x[g])
        assert np.array_equal(q[g], q1) and np.array_equal(s[g], s1)


def test_128x128_matches_blockwise_definition():
    # N = 200: the last block holds 72 rows; its amax covers only those
    x = _src((200, 384), 8)
    q, s = quant_128x128(x)
    assert s.shape == (2, 3)
    t = torch.from_numpy(x)
    for nb in range(2):
        for kb in range(3):
            blk = t[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128]
            beta = blk.abs().max() / torch.tensor(448.0)
            assert s[nb, kb] == beta.item()
            qt = (blk / beta).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128], qt)


def test_128x128_grouped_layout():
    x = _src((2, 136, 256), 9)
    q, s = quant_128x128(x)
    assert s.shape == (2, 2, 2)
    for g in range(2):
        q1, s1 = quant_128x128(x[g])
        assert np.array_equal(q[g], q1) and np.array_equal(s[g], s1)
