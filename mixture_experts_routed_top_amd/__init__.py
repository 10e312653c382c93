"""Routed-expert MoE MLP forward for MI355X (gfx950).

The compute runs in the HIP library libmoe_mi355x.so (sources in csrc/, C ABI
in include/moe_mi355x.h); this package is its ctypes binding plus a small
object (MoeLayer) that chains the calls of one forward.
"""
from ._binding import (  # noqa: F401
    ACT_RELU2, ACT_SWIGLU, DTYPE_BF16, DTYPE_FP8_BLOCK128, DTYPE_MXFP4W_MXFP8A, SCORE_SIGMOID, SCORE_SOFTMAX,
    MoeError, SortResult, lib, moe_align_sort, moe_align_sort_noalloc, moe_align_sort_workspace_bytes, moe_combine,
    moe_grouped_gemm_down, moe_grouped_gemm_relu2, moe_grouped_gemm_swiglu, moe_grouped_gemm_swiglu_h32, moe_pick_block_m, moe_quantize_fp8,
    moe_quantize_mxfp4, moe_quantize_mxfp8, moe_route, moe_route_shared, moe_sorted_capacity, moe_status_string,
    moe_backward_combine, moe_gather_rows, moe_grouped_gemm_dh, moe_grouped_gemm_dx, moe_grouped_gemm_swiglu_save,
    moe_grouped_gemm_wgrad, moe_route_backward, moe_down_combine_workspace, moe_grouped_gemm_down_combine, moe_grouped_gemm_workspace,
)
from .forward import MoeLayer, Plan, TrainBuffers  # noqa: F401
