"""Fine-grained FP8 quantisers: 1x128 per-row groups (activations) and
128x128 blocks (weights).

Lesson 13, Fig. 13-1 and the practice exercise's input description: an
activation row gets one fp32 scale per 128 consecutive K elements, equal to the
group's largest magnitude divided by 448 (the e4m3 maximum); a weight gets one
fp32 scale per 128 (output channels) x 128 (K) block.  The quantised value is
the element divided by its scale, encoded to e4m3.

Readings taken where the pages are silent:
* alpha = fl32(amax / 448) with IEEE fp32 division, and q = enc(fl32(x / alpha))
  by division (not multiplication by a reciprocal), so the result is unique and
  bit-reproducible;
* a group whose amax is zero (or whose amax / 448 underflows to zero) gets
  alpha = 1.0 and codes +-0 with the input's sign -- parity unpinned: no page
  fixes this case, it is this library's convention;
* when N is not a multiple of 128 the last weight block holds only the rows
  that exist, and its amax is taken over those rows;
* non-finite inputs are outside the contract.

Scale layouts (deep-dive blog, section 3: the activation scale tensor is stored
MN-major; the exercise gives the logical shapes [M, K/128] and
[N/128, K/128]):
* activation scales: [G][K/128][M] fp32 (M contiguous);
* weight scales:     [G][ceil(N/128)][K/128] fp32 (K/128 contiguous).
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode_e4m3

_F32_MAX = np.float32(E4M3_MAX)


def _alpha_from_amax(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(under="ignore"):
        a = (amax / _F32_MAX).astype(np.float32)  # IEEE fp32 division
    return np.where(a == 0, np.float32(1.0), a).astype(np.float32)


def quant_1x128(x: np.ndarray):
    """x: fp32 [M, K] or [G, M, K] -> (q uint8 same shape, sfa fp32 [(G,) K/128, M])."""
    x = np.asarray(x, dtype=np.float32)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[None]
    G, M, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    kb = K // 128
    xg = x.reshape(G, M, kb, 128)
    amax = np.max(np.abs(xg), axis=3)  # [G, M, kb], exact
    alpha = _alpha_from_amax(amax)  # [G, M, kb]
    y = (xg / alpha[..., None]).astype(np.float32)  # IEEE fp32 division per element
    q = encode_e4m3(y).reshape(G, M, K)
    sfa = np.ascontiguousarray(np.transpose(alpha, (0, 2, 1)))  # [G, kb, M]
    if squeeze:
        return q[0], sfa[0]
    return q, sfa


def quant_128x128(x: np.ndarray):
    """x: fp32 [N, K] or [G, N, K] -> (q uint8 same shape, sfb fp32 [(G,) ceil(N/128), K/128])."""
    x = np.asarray(x, dtype=np.float32)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[None]
    G, N, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    kb = K // 128
    nb = (N + 127) // 128
    q = np.empty((G, N, K), dtype=np.uint8)
    sfb = np.empty((G, nb, kb), dtype=np.float32)
    for b in range(nb):
        r0, r1 = 128 * b, min(128 * b + 128, N)
        blk = x[:, r0:r1, :].reshape(G, r1 - r0, kb, 128)
        amax = np.max(np.abs(blk), axis=(1, 3))  # [G, kb], over existing rows only
        beta = _alpha_from_amax(amax)
        sfb[:, b, :] = beta
        y = (blk / beta[:, None, :, None]).astype(np.float32)
        q[:, r0:r1, :] = encode_e4m3(y).reshape(G, r1 - r0, K)
    if squeeze:
        return q[0], sfb[0]
    return q, sfb
