"""CPU oracle for DDTree tree verification: test infrastructure, never the product path."""
from .ddtree_oracle import (build_mask_ref, build_tree_ref, compact_kv_ref, greedy_accept_ref, rope_inv_freq,
                            rope_neox_ref, target_argmax_ref, tree_is_valid,
                            verify_attn_ref, visible_nodes)

__all__ = ["build_mask_ref", "build_tree_ref", "compact_kv_ref", "greedy_accept_ref", "rope_inv_freq", "rope_neox_ref", "target_argmax_ref", "tree_is_valid", "verify_attn_ref",
           "visible_nodes"]
