"""Float64 CPU oracle of the fused MoE layer. Test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
"""
from .moe_oracle import (topk_select, renormalised_weights, route, sigmoid, silu, dsilu,
                         expert_forward, expert_forward_q, forward, backward, router_grad, router_forward,
                         router_backward, token_rows,
                         expert_grads, rel_frobenius)
from . import mx
