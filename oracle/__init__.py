"""CPU oracle of the DeepSeekMoE layer forward pass -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it; the product path fails loudly when its compiled
library is missing instead of falling back to anything here.
"""
from .moe_oracle import (Dispatch, Routing, activated_macs_per_token, bias_update, dispatch,
                         expert_flops_per_token, gate_logits, gate_scores,
                         group_scores, moe_forward, moe_forward_bruteforce,
                         route, select_experts, silu, swiglu_ffn)
from .moe_backward import (Grads, dsilu, exact_scores, expert_backward, moe_backward,
                           moe_forward_exact)

__all__ = [
    "Dispatch", "Routing", "activated_macs_per_token", "bias_update", "dispatch",
    "expert_flops_per_token", "gate_logits", "gate_scores", "group_scores",
    "moe_forward", "moe_forward_bruteforce", "route", "select_experts", "silu",
    "swiglu_ffn", "Grads", "dsilu", "exact_scores", "expert_backward", "moe_backward",
    "moe_forward_exact",
]
