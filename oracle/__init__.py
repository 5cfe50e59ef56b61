"""CPU oracle of the sparse-MoE FFN layer forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library and
never imports it.  Every function is float64 numpy (``moe_ref``, and
``mxfp8`` for the MXFP8 expert path) or pure Python (``brute``); see each
module's header for the passages it follows.
"""
from .moe_ref import (ACTIVATIONS, TIE_EPS, ExpertChoice, ExpertChoiceRef, MoERef, aux_loss, capacity_of,
                      capacity_ranks, expert_choice_capacity, expert_counts, expert_ffn, gelu,
                      is_valid_expert_choice, is_valid_topk, moe_forward_expert_choice_ref, moe_forward_ref,
                      renormalised_weights, router_logits, router_z_loss,
                      select_expert_choice, select_topk, selection_keys, silu, softmax, widen)

__all__ = ["ACTIVATIONS", "TIE_EPS", "ExpertChoice", "ExpertChoiceRef", "MoERef", "expert_choice_capacity",
           "is_valid_expert_choice", "moe_forward_expert_choice_ref", "select_expert_choice", "aux_loss", "capacity_of", "capacity_ranks",
           "expert_counts", "expert_ffn", "gelu", "is_valid_topk", "moe_forward_ref",
           "renormalised_weights", "router_logits", "router_z_loss",
           "select_topk", "selection_keys", "silu", "softmax", "widen"]
