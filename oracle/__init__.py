"""CPU oracle of the MoE layer hot path (float64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and
by the bench's CPU-baseline leg, never by the HIP library.  It shares no code
with that library.
"""
from .moe import (  # noqa: F401
    router_logits, topk_experts, softmax_probs, gate_weights, expert_counts,
    dispatch_permutation, dispatch_rows, silu, expert_ffn, combine, combine_backward,
    gate_backward, expert_ffn_backward, dispatch_router_backward, moe_forward,
    moe_backward, maxvio, load_entropy,
)
from .mod import mod_scores, mod_keep, mod_merge, mod_backward  # noqa: F401
