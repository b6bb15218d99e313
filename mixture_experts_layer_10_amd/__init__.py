"""MI355X (gfx950) MoE layer forward: HIP kernels behind a C ABI (libmoe.so).

The Python side is argument marshalling only (see binding.py); build the
library with `python -m mixture_experts_layer_10_amd.build`.
"""
from .binding import (  # noqa: F401
    ABI_VERSION, Config, Weights, MoEError, lib, status_string, make_config, config_from_workload,
    validate_config, workspace_bytes, workspace, make_weights, moe_router_gemm, moe_route,
    moe_dispatch, moe_expert_ffn, moe_combine, moe_forward, moe_forward_noalloc, NOALLOC_SCRATCH_BYTES, moe_dispatch_errors,
    packed_weights_bytes, moe_prepack_weights,
    moe_quantize_fp8, moe_quantize_mx, moe_expert_load,
    moe_eplb_plan,
    LIB_PATH,
    SCORE_SOFTMAX, SCORE_SIGMOID, DTYPE_F32, DTYPE_BF16, DTYPE_FP8, DTYPE_MXFP4,
    STAGES, profile_enable, profile_reset, profile_query, profile_select, mfma_loop, stream_read,
)
