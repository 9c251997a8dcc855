"""CPU oracle of the sparse MoE layer forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (capacity, capacity_drop, combine, dispatch, expert_rows_ffn, expert_choice_capacity,  # noqa: F401
                         expert_choice_select, layer_forward, rexp, route, router_logits,
                         routing_score32, routing_stats, shared_expert, silu, softmax_rows,
                         swiglu_ffn, topk_gates, topk_select, widen)
