"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench."""
from .gen import (CONFIGS, DraftCandidates, Workload, bf16_bits, bf16_to_f32, bounded_tree, chain_tree, make_accept_draws, make_config,
                  make_draft_candidates, make_workload, restrict, to_f32, uniform_tree)

__all__ = ["CONFIGS", "DraftCandidates", "Workload", "bf16_bits", "bf16_to_f32", "bounded_tree", "chain_tree", "make_accept_draws", "make_config",
           "make_draft_candidates", "make_workload", "restrict", "to_f32", "uniform_tree"]
