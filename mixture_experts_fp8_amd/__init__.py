"""Routed FP8 Mixture-of-Experts expert step for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
include/moe_fp8.h (library: mixture_experts_fp8_amd/lib/libmoe_fp8.so); this package
only holds those sources (csrc/), the build script and a thin ctypes binding whose
functions carry the C entry points' names.
"""
from .binding import (  # noqa: F401
    MoeError, MoeFused, PackedWeights, Prelude, RouteParams, lib, moe_combine, moe_fused,
    moe_grouped_ffn, moe_last_error, moe_prepack_weights, moe_quant_act, moe_quant_weight_blocks,
    moe_route, moe_workspace_size, route_params, moe_quant_act_mx, moe_quant_weight_mx, moe_prepack_weights_mx,
    pack_weights_mx, MOE_QUANT_FP8_BLOCK128, MOE_QUANT_MXFP8, MOE_QUANT_W4A8, MOE_QUANT_W8A16, MOE_WFMT_E4M3, MOE_WFMT_E2M1,
    QUANT_SCHEMES, MOE_FUSED_EXPERT_OUT_BF16, MOE_FUSED_SHARED_EXPERT, moe_fused_static, MOE_STATIC_SCRATCH_BYTES,
)
