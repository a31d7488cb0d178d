"""MI355X-native (gfx950) block-scaled FP8 GEMM with MoE grouped forms.

The compute path is the HIP library ``libdg_mi355x.so`` (C ABI: include/dg.h);
``dg`` is its argument-marshalling binding.  The library is loaded on first
use; importing the package alone does not need a GPU.
"""

from .dg import (  # noqa: F401
    DG_OP_BF16_GEMM_NT,
    DG_OP_CONTIGUOUS,
    DG_OP_GEMM_NT,
    DG_OP_GEMM_NT_UE8M0,
    DG_OP_K_GROUPED,
    DG_OP_MASKED,
    DGError,
    dg_bf16_gemm_nt,
    dg_describe_plan,
    dg_fp8_gemm_nt,
    dg_fp8_gemm_nt_acc,
    dg_fp8_gemm_nt_ue8m0,
    dg_get_m_alignment_for_contiguous_layout,
    dg_get_num_cus,
    dg_get_workspace_size,
    dg_k_grouped_fp8_gemm_nt_contiguous,
    dg_m_grouped_fp8_gemm_nt_contiguous,
    dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0,
    dg_m_grouped_fp8_gemm_nt_masked,
    dg_m_grouped_fp8_gemm_nt_masked_ue8m0,
    dg_quant_128x128,
    dg_quant_128x128_ue8m0,
    dg_quant_1x128,
    dg_quant_1x128_ue8m0,
    dg_set_num_cus,
    dg_version,
    load_library,
)

__version__ = "0.2.0"
