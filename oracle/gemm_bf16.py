"""BF16 dense GEMM, D = A . B^T rounded to bf16.  TEST INFRASTRUCTURE ONLY.

The pages put a BF16 GEMM beside the FP8 one: BF16 is among the library's
precisions ("DeepGEMM architecture deep dive", section 1, the overview
table; the Ascend 950 DeepGEMM article's list of kernels), and the Ascend
article measures a BF16 dense GEMM at 4096 x 7168 x 16384 (benchmarks
section).  Same NT layout as the FP8 path
(deep dive, section 3: D = A @ B^T with both operands K-contiguous), no
scales, output bf16.

Operands arrive as uint16 bf16 bit patterns.  Every product of two bf16
values is exact in fp64 (8 + 8 significant bits); the sum over K uses numpy's
fp64 matrix product (a library step), whose rounding error is many orders of
magnitude below half a bf16 ulp, and the result is rounded once to bf16 with
round-to-nearest-even (the same epilogue reading as the FP8 path).
"""

import numpy as np

from .bf16 import bf16_bits_to_f64, bf16_rne_bits


def gemm_bf16_nt(a_bits, b_bits) -> np.ndarray:
    """a_bits [M, K], b_bits [N, K] (uint16 bf16) -> D [M, N] uint16 bf16 bits."""
    a = bf16_bits_to_f64(np.asarray(a_bits, dtype=np.uint16))
    b = bf16_bits_to_f64(np.asarray(b_bits, dtype=np.uint16))
    return bf16_rne_bits(a @ b.T)
