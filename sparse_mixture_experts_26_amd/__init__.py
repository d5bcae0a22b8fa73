"""MI355X (gfx950) sparse Mixture-of-Experts layer forward.

The compute path is libmoe.so (HIP kernels behind a C ABI, include/moe.h);
this package is its ctypes binding.  Importing it loads nothing; the library
is loaded on first use and a missing build raises instead of falling back.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, MoeAux, MoeConfig, MoeError, MoeWeights, lib, make_config,
    moe_capacity, moe_combine, moe_dispatch, moe_expert_down, moe_expert_ffn, moe_expert_up,
    moe_layer_forward, moe_route, moe_routed_rows_bound, moe_status_string,
    moe_workspace_bytes, status_string, moe_router_diagnostics, moe_expert_choice,
    moe_combine_expert_choice, moe_dispatch_reroute, moe_backward_workspace_bytes,
    moe_layer_backward, MoeGrads, moe_route_launch_shape, moe_layer_forward_noalloc,
    MOE_NOALLOC_SCRATCH_BYTES,
    MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL,
    MOE_ERR_HIP, MOE_F32, MOE_BF16, MOE_ACT_GELU, MOE_ACT_RELU, MOE_ACT_SWIGLU,
    MOE_ROUTE_TOKEN_CHOICE, MOE_ROUTE_EXPERT_CHOICE, MOE_OVERFLOW_DROP, MOE_OVERFLOW_REROUTE,
)
