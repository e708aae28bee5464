"""MI355X (gfx950) MoE token routing with equal-cost load-balancing statistics.

The compute path is the HIP library ``_lib/libmoe_route.so`` behind the C ABI
of ``include/moe_route.h``; this package is its thin ctypes binding (same
names) plus the seeded synthetic workloads used by the tests and benchmark.
"""
from ._binding import (  # noqa: F401
    MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_SCRATCH, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_OK,
    MOE_ROUTE_SCRATCH_BYTES,
    MOE_RENORM_TOPK, MOE_ROUTE_MAX_E, MOE_ROUTE_MAX_K, MOE_SAVE_ROW_STATS,
    MOE_MULTI_KERNEL, MOE_P_MASKED, MOE_SELECT_BIAS, MOE_STATUS_INTERNAL, MOE_STATUS_NONFINITE, MOE_WRITE_INV_PERM, MoeRouteError,
    alloc_outputs, alloc_workspace, load, make_params, moe_eplb_plan, moe_gate_backward,
    moe_gate_backward_workspace_size, moe_route, moe_route_backward, moe_route_noalloc,
    moe_route_bias_update, moe_route_capacity, moe_route_with_bias_update, moe_route_params, moe_route_strerror, moe_route_workspace_size,
    moe_sinkhorn_plan)
