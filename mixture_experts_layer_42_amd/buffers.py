"""Device-memory helpers around the C ABI (allocation and upload only)."""
from __future__ import annotations

import numpy as np

from ._lib import (MOE_BF16, MOE_EXPERT_CHOICE, MOE_F32, MOE_TOKEN_CHOICE, make_problem,
                   make_routing)


def problem_of(cfg):
    """moe_problem from any object with the fields T, d_model, E, k, d_ff, d_ff_shared,
    routing ("token"/"expert"), gamma, renorm_topk, dtype ("bf16"/"f32") and optionally
    y_dtype ("bf16"/"f32"/"" = same as dtype), expand_m and cap_groups (default 0)."""
    y_dt = getattr(cfg, "y_dtype", "") or cfg.dtype
    return make_problem(cfg.T, cfg.d_model, cfg.E, cfg.k, cfg.d_ff, cfg.d_ff_shared,
                        MOE_EXPERT_CHOICE if cfg.routing == "expert" else MOE_TOKEN_CHOICE,
                        float(cfg.gamma), int(bool(cfg.renorm_topk)),
                        MOE_BF16 if cfg.dtype == "bf16" else MOE_F32,
                        MOE_BF16 if y_dt == "bf16" else MOE_F32,
                        int(getattr(cfg, "expand_m", 0) or 0),
                        int(getattr(cfg, "cap_groups", 0) or 0))


def device_tensor(a, device="cuda"):
    """Upload a host array. uint16 arrays are bfloat16 bit patterns."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class RoutingBuffers:
    """Caller-owned routing arrays for one problem (all on `device`)."""

    def __init__(self, problem, device="cuda"):
        import torch
        T, E, k = problem.T, problem.E, problem.k
        S = k + problem.expand_m          # slots per token (extra Expanded Drop candidates)
        R = T * k
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty(T, E, dtype=f32, device=device)
        self.topk_ids = torch.empty(T, S, dtype=i32, device=device)
        self.topk_w = torch.empty(T, S, dtype=f32, device=device)
        self.kept = torch.empty(T, S, dtype=torch.uint8, device=device)
        self.counts = torch.empty(E, dtype=i32, device=device)
        self.offsets = torch.empty(E + 1, dtype=i32, device=device)
        self.perm_token = torch.empty(R, dtype=i32, device=device)
        self.perm_w = torch.empty(R, dtype=f32, device=device)
        self.tok_ptr = torch.empty(T + 1, dtype=i32, device=device)
        self.tok_pos = torch.empty(R, dtype=i32, device=device)
        self.struct = make_routing(**{n: getattr(self, n) for n in (
            "logits", "topk_ids", "topk_w", "kept", "counts", "offsets", "perm_token", "perm_w",
            "tok_ptr", "tok_pos")})

    def host(self):
        """Copies of every array as numpy (synchronises)."""
        return {n: getattr(self, n).cpu().numpy() for n in (
            "logits", "topk_ids", "topk_w", "kept", "counts", "offsets", "perm_token", "perm_w",
            "tok_ptr", "tok_pos")}
