"""MI355X-native forward pass of one sparse Mixture-of-Experts layer.

The computation lives in ``libmoe.so`` (hand-written HIP for gfx950 behind a C ABI,
``include/moe.h``); this package is its thin Python binding. PyTorch is used only
for device memory and streams.

    import mixture_experts_layer_42_amd as moe
    prob = moe.make_problem(T, d_model, E, k, d_ff, dtype=moe.MOE_BF16)
    ws = torch.empty(moe.moe_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    moe.moe_layer_forward(prob, x, w_router, bias, w_gate, w_up, w_down, None, None, None,
                          y, None, ws, ws.numel())
"""
from ._lib import (EXPORTED, LIB_PATH, MOE_BF16, MOE_ERR_HIP, MOE_ERR_INVALID_ARG,  # noqa: F401
                   MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_EXPERT_CHOICE, MOE_F32, MOE_OK,
                   MOE_ROUTE_LOGITS_IN, MOE_STAGE_COUNT, MOE_TOKEN_CHOICE, STAGE_NAMES, MoEError,
                   load, make_problem, make_routing, moe_combine, moe_dispatch, moe_expert_ffn,
                   moe_layer_forward, moe_layer_forward_traced, moe_problem, moe_route,
                   moe_route_noalloc, moe_routing, moe_routing_stats, moe_workspace_bytes,
                   status_str)
from .buffers import RoutingBuffers, device_tensor, problem_of  # noqa: F401
