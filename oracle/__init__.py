"""fp64 CPU oracle of the sparse-MoE decode step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (E2M1, adjacent_gaps, bf16_to_f64, e2m1_value, e8m0_value,
                         expert_activation, expert_ffn, f64_to_bf16, group_by_expert,
                         moe_layer, moe_stack, mx_decode, rmsnorm_bf16, router_logits,
                         silu, topk_gap, topk_select, topk_weights)
