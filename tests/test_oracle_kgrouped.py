"""Pins of the K-grouped contiguous oracle (oracle.k_grouped_contiguous) to
things other than itself: exact rational brute force with its own segment
walk, integer exactness against a plain matmul per segment, the dense
oracle on a single segment whose per-row weight scales are constant over
128-row blocks, empty groups, and planted mistakes (shifted segment, scales
of the wrong block, swapped groups, per-block instead of per-row scales,
C dropped) that the exact pin must catch."""

import numpy as np
import pytest

from oracle import decode_e4m3, encode_e4m3, gemm_nt_c, k_grouped_contiguous
from oracle.exact import k_grouped_exact
from oracle.gemm_kgrouped import segment_blocks

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _case(M, N, ks, seed, with_c=True):
    rng = np.random.default_rng(seed)
    K = int(sum(ks))
    a = FINITE[rng.integers(0, FINITE.size, (M, K))]
    b = FINITE[rng.integers(0, FINITE.size, (N, K))]
    sfa = rng.uniform(0.25, 4, (K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.25, 4, (K // 128, N)).astype(np.float32)
    c = (rng.standard_normal((len(ks), M, N)) * 1e3).astype(np.float32) if with_c else None
    return a, sfa, b, sfb, c


@pytest.mark.parametrize("M,N,ks,seed,with_c", [
    (2, 3, [128, 256], 1, True),
    (3, 2, [256, 0, 128], 2, True),
    (2, 2, [0, 128, 128, 0], 3, False),
])
def test_k_grouped_equals_exact_rational(M, N, ks, seed, with_c):
    a, sfa, b, sfb, c = _case(M, N, ks, seed, with_c)
    got = k_grouped_contiguous(a, sfa, b, sfb, ks, c)
    ref = k_grouped_exact(a, sfa, b, sfb, ks, c)
    assert got.shape == (len(ks), M, N)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_k_grouped_integer_inputs_exact():
    rng = np.random.default_rng(4)
    M, N, ks = 6, 5, [384, 128, 0, 256]
    K = sum(ks)
    qa = encode_e4m3(rng.integers(-12, 12, (M, K)).astype(np.float32))
    qb = encode_e4m3(rng.integers(-12, 12, (N, K)).astype(np.float32))
    c = rng.integers(-1000, 1000, (len(ks), M, N)).astype(np.float32)
    ones_a = np.ones((K // 128, M), np.float32)
    ones_b = np.ones((K // 128, N), np.float32)
    a, b = decode_e4m3(qa), decode_e4m3(qb)
    got = k_grouped_contiguous(qa, ones_a, qb, ones_b, ks, c)
    lo = 0
    for g, k in enumerate(ks):
        ref = a[:, lo:lo + k] @ b[:, lo:lo + k].T + c[g]
        assert np.array_equal(got[g], ref.astype(np.float32)), g
        lo += k


def test_single_segment_reduces_to_dense_oracle():
    # per-row weight scales constant over each 128-row block are the dense
    # form's 128x128 block scales
    rng = np.random.default_rng(5)
    M, N, K = 7, 200, 384
    a = FINITE[rng.integers(0, FINITE.size, (M, K))]
    b = FINITE[rng.integers(0, FINITE.size, (N, K))]
    sfa = rng.uniform(0.5, 2, (K // 128, M)).astype(np.float32)
    sfb_blk = rng.uniform(0.5, 2, ((N + 127) // 128, K // 128)).astype(np.float32)
    sfb_row = sfb_blk[np.arange(N) // 128].T.copy()  # [K/128, N]
    c = rng.standard_normal((M, N)).astype(np.float32)
    got = k_grouped_contiguous(a, sfa, b, sfb_row, [K], c[None])
    assert np.array_equal(got[0].view(np.uint32), gemm_nt_c(a, sfa, b, sfb_blk, c).view(np.uint32))


def test_empty_groups_and_unused_tail():
    a, sfa, b, sfb, c = _case(3, 4, [256, 128], 6)
    # group 1 empty: D[1] = C[1] exactly; the last 128 K positions belong to no group
    got = k_grouped_contiguous(a, sfa, b, sfb, [256, 0], c)
    assert np.array_equal(got[1], c[1])
    full = k_grouped_contiguous(a, sfa, b, sfb, [256, 128], c)
    assert np.array_equal(got[0], full[0])
    assert np.array_equal(k_grouped_contiguous(a, sfa, b, sfb, [0, 0], None), np.zeros((2, 3, 4), np.float32))


def test_segment_validation():
    assert segment_blocks([128, 0, 256], 512) == [(0, 1), (1, 0), (1, 2)]
    for bad in ([100], [-128], [256, 384]):
        with pytest.raises(ValueError):
            segment_blocks(bad, 512)


@pytest.mark.parametrize("mistake", ["shifted_segment", "scale_of_next_block", "groups_swapped",
                                     "block_scale_not_row", "c_dropped"])
def test_planted_mistakes_fail_the_exact_pin(mistake):
    M, N, ks = 2, 3, [128, 256]
    a, sfa, b, sfb, c = _case(M, N, ks, 7)
    K = sum(ks)
    A, B = decode_e4m3(a), decode_e4m3(b)
    sa, sb = sfa.astype(np.float64), sfb.astype(np.float64)

    def grouped(blocks_of, scale_a, scale_b, add_c=True):
        out = np.zeros((len(ks), M, N))
        for g, blks in enumerate(blocks_of):
            for blk in blks:
                cols = slice(128 * blk, 128 * blk + 128)
                out[g] += scale_a(blk)[:, None] * scale_b(blk)[None, :] * (A[:, cols] @ B[:, cols].T)
        if add_c:
            out += c.astype(np.float64)
        return out.astype(np.float32)

    right = [[0], [1, 2]]
    if mistake == "shifted_segment":
        bad = grouped([[0], [0, 1]], lambda k: sa[k], lambda k: sb[k])
    elif mistake == "scale_of_next_block":
        bad = grouped(right, lambda k: sa[k], lambda k: sb[(k + 1) % (K // 128)])
    elif mistake == "groups_swapped":
        bad = grouped([[1, 2], [0]], lambda k: sa[k], lambda k: sb[k])
    elif mistake == "block_scale_not_row":
        bad = grouped(right, lambda k: sa[k], lambda k: np.full(N, sb[k][0]))
    else:
        bad = grouped(right, lambda k: sa[k], lambda k: sb[k], add_c=False)
    ref = k_grouped_exact(a, sfa, b, sfb, ks, c)
    assert np.array_equal(grouped(right, lambda k: sa[k], lambda k: sb[k]).view(np.uint32), ref.view(np.uint32))
    assert not np.array_equal(bad.view(np.uint32), ref.view(np.uint32))
