"""MI355X (gfx950) MoE FFN hot path: routing, permutation, grouped SwiGLU /
down GEMMs, combine and the FFN backward, behind the C ABI of include/moe.h.

The Python names mirror the C entry points (see binding.py); the HIP library
libmoe.so is loaded on first use and its absence is an error.
"""
from .binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MoEConfig,
    MoEError,
    MoEHipError,
    MoEInvalidArgument,
    MoEUnsupported,
    MoEWorkspaceError,
    alloc_backward,
    alloc_forward,
    load_library,
    moe_backward,
    moe_combine,
    moe_combine_bwd,
    moe_route_bwd,
    moe_grouped_swiglu_gemm_gather,
    moe_grouped_swiglu_gemm_weighted,
    moe_grouped_down_gemm_weighted,
    moe_forward,
    moe_forward_noalloc,
    moe_grouped_down_bwd,
    moe_grouped_down_gemm,
    moe_grouped_swiglu_bwd,
    moe_grouped_swiglu_gemm,
    moe_permute,
    moe_permute_bwd,
    moe_quantize_mxfp4,
    moe_quantize_mxfp8,
    moe_route,
    rows_capacity,
    workspace_size,
    backward_workspace_size,
)
