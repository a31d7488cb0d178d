"""K-grouped contiguous FP8 GEMM (the MoE weight-gradient form), plain and
slow, in fp64.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("DeepGEMM architecture deep dive", blog.123qwe.co.kr,
section 3, the table of the three grouped GEMM families): the K-grouped
contiguous family groups along K with M and N the same for every group, and
serves the backward pass of MoE weights; section 3 also states that every
GEMM of the library is D = C + A @ B, NT by default, and that contiguous
layouts align each expert's segment to the block size
(get_mk_alignment_for_contiguous_layout, "mk": the alignment holds for M and
for K).

Readings where the pages are silent (each one also stated where the layout
is declared):
* group g owns the K range [k_0 + ... + k_{g-1}, k_0 + ... + k_g) of both
  operands, ks[g] a multiple of 128 (zero allowed: that expert received no
  tokens); positions past the last segment belong to no group;
* both operands are activations of the backward pass (output gradient and
  layer input, transposed so that tokens run along K), so both carry the
  activation granularity of Lesson 13, Fig. 13-1: one fp32 scale per row
  per 128 K elements, MN-major ([K/128, M] and [K/128, N]);
* the per-128-K promotion of Lesson 13, Fig. 13-1 applies unchanged inside
  each segment: a block's exact partial is multiplied by alpha[row] *
  beta[column] of that block and added into the group's accumulator, blocks
  ascending;
* the output is the fp32 accumulating form of section 3, one [M, N] matrix
  per group: D[g] = C[g] + sum over the group's blocks, rounded once to fp32
  (C absent: zero).

Exactness is that of ``gemm.py``: each 128-element partial of decoded e4m3
values is exact in fp64 (a BLAS matmul is a valid primitive for it), the
product of two fp32 scales is exact, and only the running fp64 sum and the
final fp32 conversion round.
"""

import numpy as np

from .e4m3 import decode_e4m3


def segment_blocks(ks, K):
    """(first K block, number of K blocks) of every group, from ks (elements).

    Raises ValueError unless every ks[g] is a non-negative multiple of 128 and
    the segments fit in K."""
    ks = [int(k) for k in np.asarray(ks).reshape(-1)]
    out = []
    lo = 0
    for k in ks:
        if k < 0 or k % 128:
            raise ValueError("every ks[g] must be a non-negative multiple of 128")
        out.append((lo // 128, k // 128))
        lo += k
    if lo > K:
        raise ValueError("segments exceed K")
    return out


def k_grouped_contiguous(a_codes, sfa, b_codes, sfb, ks, c) -> np.ndarray:
    """fp32 [G, M, N] of D[g] = C[g] + A[:, seg_g] . B[:, seg_g]^T.

    a_codes: uint8 [M, K]; sfa: fp32 [K/128, M] (per row and 128-K block)
    b_codes: uint8 [N, K]; sfb: fp32 [K/128, N] (per row and 128-K block)
    ks: int [G] segment lengths; c: fp32 [G, M, N] or None (zero)
    """
    a = decode_e4m3(a_codes)
    b = decode_e4m3(b_codes)
    M, K = a.shape
    N, Kb = b.shape
    if K != Kb or K % 128:
        raise ValueError("K mismatch or K not a multiple of 128")
    sfa = np.asarray(sfa, dtype=np.float32).astype(np.float64)
    sfb = np.asarray(sfb, dtype=np.float32).astype(np.float64)
    if sfa.shape != (K // 128, M) or sfb.shape != (K // 128, N):
        raise ValueError("scale tensor shape mismatch")
    segs = segment_blocks(ks, K)
    G = len(segs)
    out = np.zeros((G, M, N), dtype=np.float64)
    for g, (blk0, nblk) in enumerate(segs):
        for blk in range(blk0, blk0 + nblk):
            cols = slice(128 * blk, 128 * blk + 128)
            partial = a[:, cols] @ b[:, cols].T  # exact
            out[g] += (sfa[blk][:, None] * sfb[blk][None, :]) * partial
    if c is not None:
        out += np.asarray(c, dtype=np.float32).astype(np.float64)
    return out.astype(np.float32)
