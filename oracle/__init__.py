"""CPU oracle for block-scaled FP8 GEMM (dense, M-grouped contiguous, M-grouped
masked, K-grouped contiguous, the fp32 accumulating form, UE8M0 scales) and the
BF16 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP kernels under ``moe_grouped_matmul_amd/csrc``.

What it computes comes from these pages:

* Lesson 13, "DeepSeek DeepGEMM core architecture and Hopper FP8 operator
  breakdown" (hpc.payai.win): Fig. 13-1 (1x128 activation scales, 128x128
  weight scales, per-128-K promotion and its closed-form equation),
  Fig. 13-3 (contiguous and masked MoE layouts), the practice exercise
  (dequantise-first reference vs promoted form) and the Q1/Q3 answers.
* "DeepGEMM architecture deep dive" (blog.123qwe.co.kr), section 3
  (NT layout, D = A @ B^T, scale layouts, M alignment of contiguous groups).

Everything is evaluated so that each step before the final bf16 rounding is
exact or within about 1e-16 relative: e4m3 values are decoded from the format
definition, each 128-wide K partial sum is formed in fp64 (exact, see
``gemm.py``), scaled and accumulated in fp64, and rounded once to bf16 with
round-to-nearest-even.

Parity pins (tests/test_oracle_*.py) tie every function here to something
other than itself: torch's independent float8/bfloat16 casts, exact rational
brute force (``exact.py``), closed forms, integer exactness, linearity and the
page's own worked exercise.  Conventions the pages leave open and that no
external source fixes -- the all-zero quantisation group (alpha := 1) and the
sign of zero codes -- are marked "parity unpinned" where they are defined.
"""

from .e4m3 import E4M3_MAX, decode_e4m3, encode_e4m3
from .bf16 import bf16_rne_bits, bf16_bits_to_f64
from .quant import quant_1x128, quant_128x128
from .gemm_bf16 import gemm_bf16_nt
from .gemm_kgrouped import k_grouped_contiguous
from .ue8m0 import (
    gemm_nt_ue8m0,
    grouped_contiguous_ue8m0,
    grouped_masked_ue8m0,
    quant_1x128_ue8m0,
    quant_128x128_ue8m0,
)
from .gemm import (
    gemm_nt_acc,
    gemm_nt,
    gemm_nt_c,
    grouped_contiguous,
    grouped_masked,
)

__all__ = [
    "E4M3_MAX",
    "decode_e4m3",
    "encode_e4m3",
    "bf16_rne_bits",
    "bf16_bits_to_f64",
    "quant_1x128",
    "quant_128x128",
    "gemm_nt_acc",
    "gemm_nt",
    "gemm_nt_c",
    "grouped_contiguous",
    "grouped_masked",
    "gemm_bf16_nt",
    "k_grouped_contiguous",
    "quant_1x128_ue8m0",
    "quant_128x128_ue8m0",
    "gemm_nt_ue8m0",
    "grouped_contiguous_ue8m0",
    "grouped_masked_ue8m0",
]
