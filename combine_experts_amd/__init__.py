"""MI355X-native (gfx950) MoE layer: route, one-sided dispatch, grouped SwiGLU
expert GEMMs with the shared expert, and a weighted combine, all in
hand-written HIP kernels behind the C ABI of include/moe.h.

This package is the thin Python binding of that library (libmoe_hip.so, built
in-tree by combine_experts_amd/build.py).  Importing it loads the library and
fails with ImportError when it has not been built; there is no fallback."""
from ._binding import (  # noqa: F401
    DTYPE, LIB_PATH, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL,
    MOE_ERR_SCRATCH_LIMIT, MOE_OK, SCORE, WEIGHT, MoeConfig, MoeError, MoeWeights, load_library, make_config, make_weights,
    moe_combine, moe_dispatch, moe_dispatch_rows, moe_expert_ffn, moe_ffn_down, moe_ffn_gate_up,
    moe_ffn_workspace_size, moe_fused_supported, moe_fused_workspace_size, moe_layer, moe_layer_fused,
    moe_layer_static, moe_layer_static_max_bytes,
    moe_router_logits, moe_router_logits_ws, moe_router_workspace_size,
    moe_route, moe_route_dispatch, moe_status_string, moe_workspace_size)

load_library()
