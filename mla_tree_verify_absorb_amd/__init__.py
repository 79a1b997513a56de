"""MI355X (gfx950) DDTree tree verification: visibility mask, tree-verify MLA-absorb
attention, greedy tree accept, post-verify KV-cache compaction and the best-first
draft-tree builder and the NeoX rotary embedding at tree positions, as a C-ABI
HIP library (libddtree.so) with a thin ctypes binding."""
from ._lib import (DDTREE_BF16, DDTREE_ERR_HIP, DDTREE_ERR_INVALID_ARG, DDTREE_ERR_UNSUPPORTED,
                   DDTREE_ERR_WORKSPACE, DDTREE_F32, DDTREE_MAX_DEPTH, DDTREE_MAX_NODES, DDTREE_MAX_PROPOSALS,
                   DDTREE_NOALLOC_SCRATCH_BYTES, DDTREE_OK, ddtree_build_mask, ddtree_build_tree, ddtree_compact_kv,
                   ddtree_greedy_accept, ddtree_rope_tree, ddtree_status_string, ddtree_verify_attn, ddtree_verify_attn_auto_splits,
                   ddtree_verify_attn_noalloc, ddtree_verify_attn_workspace_size, lib, library_path)

__all__ = ["DDTREE_BF16", "DDTREE_ERR_HIP", "DDTREE_ERR_INVALID_ARG", "DDTREE_ERR_UNSUPPORTED", "DDTREE_ERR_WORKSPACE",
           "DDTREE_F32", "DDTREE_MAX_DEPTH", "DDTREE_MAX_NODES", "DDTREE_MAX_PROPOSALS", "DDTREE_NOALLOC_SCRATCH_BYTES", "DDTREE_OK",
           "ddtree_build_mask", "ddtree_build_tree", "ddtree_compact_kv", "ddtree_greedy_accept", "ddtree_rope_tree",
           "ddtree_status_string", "ddtree_verify_attn", "ddtree_verify_attn_auto_splits",
           "ddtree_verify_attn_noalloc", "ddtree_verify_attn_workspace_size", "lib", "library_path"]
