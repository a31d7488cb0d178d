"""UE8M0 (power-of-two) scale variant: quantisers, packing and the GEMM, plain
and slow.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: the scales of the block-scaled FP8 GEMM are fp32, and
newer library versions also accept UE8M0 scales (Lesson 13, hpc.payai.win,
the notes on block-wise scaling after Fig. 13-1); on the newer architecture
the scales are UE8M0 with four of them packed into one 32-bit integer
("DeepGEMM architecture deep dive", blog.123qwe.co.kr, section 3,
scaling-factor formats).  The
granularity (1x128 activations, 128x128 weights; Lesson 13, Fig. 13-1) and
the per-128-K promotion do not change; only the number format of the scale
does.

Readings where the pages are silent:
* a UE8M0 byte c is the power of two 2^(c - 127) (an unsigned exponent with
  bias 127, the E8M0 encoding); this library never produces c = 255;
* a group's scale is the smallest power of two not below amax / 448, so that
  no element of the group saturates: c = 127 + min{e : 448 * 2^e >= amax},
  clamped to [0, 254];
* an all-zero group gets c = 127 (scale 1), as the fp32 form's alpha := 1 --
  parity unpinned, this library's convention;
* the quantised value is e4m3_RNE(x / 2^(c - 127)); the division by a power
  of two is exact, so the bytes are unique;
* packing: four consecutive K blocks' codes share one int32, block 4w + j in
  byte j (bits 8j .. 8j + 7), unused bytes zero.  Activation scales keep the
  MN-major layout of the fp32 form, [ceil(KB/4)][M]; weight scales are
  [ceil(N/128)][ceil(KB/4)] (KB = K / 128).
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode_e4m3
from .gemm import gemm_nt, grouped_contiguous, grouped_masked


def ue8m0_code(amax) -> np.ndarray:
    """Code of the smallest power of two >= amax / 448 (amax fp32 >= 0)."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    out = np.full(a.shape, 127, dtype=np.int64)
    pos = a > 0
    if np.any(pos):
        ap = a[pos]
        with np.errstate(divide="ignore"):
            e = np.ceil(np.log2(ap / E4M3_MAX)).astype(np.int64)
        # exact corrections: 448 * 2^e is exact in fp64 for the exponents here
        for _ in range(2):
            e = np.where(np.ldexp(E4M3_MAX, e) < ap, e + 1, e)
            e = np.where(np.ldexp(E4M3_MAX, e - 1) >= ap, e - 1, e)
        out[pos] = np.clip(e + 127, 0, 254)
    return out.astype(np.uint8)


def ue8m0_value(codes) -> np.ndarray:
    """fp32 value 2^(c - 127) of UE8M0 codes (c < 255)."""
    c = np.asarray(codes, dtype=np.int64)
    return np.ldexp(np.float64(1.0), c - 127).astype(np.float32)


def _quant(xg, code):
    # xg [..., 128] fp32; code [...]: q = e4m3_RNE(x * 2^-(c - 127)), exact scaling
    y = np.ldexp(xg.astype(np.float64), -(code.astype(np.int64) - 127)[..., None]).astype(np.float32)
    return encode_e4m3(y)


def pack_k(codes) -> np.ndarray:
    """Pack codes [..., KB] (uint8) into int32 [..., ceil(KB/4)], block 4w + j in byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    kb = c.shape[-1]
    w = (kb + 3) // 4
    padded = np.zeros(c.shape[:-1] + (4 * w,), dtype=np.uint32)
    padded[..., :kb] = c
    p = padded.reshape(c.shape[:-1] + (w, 4))
    return (p[..., 0] | (p[..., 1] << 8) | (p[..., 2] << 16) | (p[..., 3] << 24)).astype(np.uint32).view(np.int32)


def unpack_k(words, kb) -> np.ndarray:
    """Inverse of pack_k: int32 [..., W] -> uint8 [..., kb]."""
    w = np.asarray(words).astype(np.int32).view(np.uint32)
    b = np.stack([(w >> (8 * j)) & 0xFF for j in range(4)], axis=-1).reshape(w.shape[:-1] + (4 * w.shape[-1],))
    return b[..., :kb].astype(np.uint8)


def quant_1x128_ue8m0(x: np.ndarray):
    """x fp32 [M, K] -> (q uint8 [M, K], codes uint8 [K/128, M], packed int32 [ceil(KB/4), M])."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    kb = K // 128
    xg = x.reshape(M, kb, 128)
    code = ue8m0_code(np.max(np.abs(xg), axis=2))  # [M, kb]
    q = _quant(xg, code).reshape(M, K)
    codes = np.ascontiguousarray(code.T)  # [kb, M]
    packed = np.ascontiguousarray(pack_k(code).T)  # [W, M]
    return q, codes, packed


def quant_128x128_ue8m0(x: np.ndarray):
    """x fp32 [N, K] -> (q uint8 [N, K], codes uint8 [ceil(N/128), K/128], packed int32 [ceil(N/128), ceil(KB/4)])."""
    x = np.asarray(x, dtype=np.float32)
    N, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    kb = K // 128
    nb = (N + 127) // 128
    q = np.empty((N, K), dtype=np.uint8)
    codes = np.empty((nb, kb), dtype=np.uint8)
    for b in range(nb):
        r0, r1 = 128 * b, min(128 * b + 128, N)
        blk = x[r0:r1].reshape(r1 - r0, kb, 128)
        code = ue8m0_code(np.max(np.abs(blk), axis=(0, 2)))  # [kb], over existing rows
        codes[b] = code
        q[r0:r1] = _quant(blk, np.broadcast_to(code, (r1 - r0, kb))).reshape(r1 - r0, K)
    return q, codes, pack_k(codes)


def gemm_nt_ue8m0(a_codes, sfa_packed, b_codes, sfb_packed) -> np.ndarray:
    """bf16 bits [M, N] of the promoted GEMM with UE8M0 scales: the packed codes
    decoded to their powers of two and the fp32-scale definition applied."""
    M, K = np.asarray(a_codes).shape
    N = np.asarray(b_codes).shape[0]
    kb = K // 128
    sfa = ue8m0_value(unpack_k(np.asarray(sfa_packed).T, kb).T)  # [kb, M]
    sfb = ue8m0_value(unpack_k(np.asarray(sfb_packed), kb))  # [nb, kb]
    if sfa.shape != (kb, M) or sfb.shape != ((N + 127) // 128, kb):
        raise ValueError("scale tensor shape mismatch")
    return gemm_nt(a_codes, sfa, b_codes, sfb)


def _decode_act(sfa_packed, kb):
    """Packed activation codes [..., W, rows] -> fp32 powers of two [..., kb, rows]."""
    w = np.asarray(sfa_packed)
    return ue8m0_value(np.swapaxes(unpack_k(np.swapaxes(w, -1, -2), kb), -1, -2))


def grouped_contiguous_ue8m0(a_codes, sfa_packed, b_codes, sfb_packed, m_indices, d_init) -> np.ndarray:
    """M-grouped contiguous layout with UE8M0 scales (Lesson 13, Fig. 13-3;
    deep-dive blog, section 3: the grouped GEMMs take the same scale formats):
    sfa_packed int32 [ceil(KB/4), M_total], sfb_packed int32 [G, ceil(N/128),
    ceil(KB/4)]; the codes decoded to their powers of two and the fp32-scale
    grouped definition applied (rows with an index outside [0, G) untouched)."""
    kb = np.asarray(a_codes).shape[1] // 128
    return grouped_contiguous(a_codes, _decode_act(sfa_packed, kb), b_codes,
                              ue8m0_value(unpack_k(np.asarray(sfb_packed), kb)), m_indices, d_init)


def grouped_masked_ue8m0(a_codes, sfa_packed, b_codes, sfb_packed, masked_m, d_init) -> np.ndarray:
    """M-grouped masked layout with UE8M0 scales: sfa_packed int32
    [G, ceil(KB/4), max_m], sfb_packed int32 [G, ceil(N/128), ceil(KB/4)];
    decoded, then the fp32-scale masked definition (rows at or past
    clamp(masked_m[g], 0, max_m) untouched)."""
    kb = np.asarray(a_codes).shape[2] // 128
    return grouped_masked(a_codes, _decode_act(sfa_packed, kb), b_codes,
                          ue8m0_value(unpack_k(np.asarray(sfb_packed), kb)), masked_m, d_init)
