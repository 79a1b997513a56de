"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench."""
from .gen import (CONFIGS, Workload, bf16_bits, bf16_to_f32, bounded_tree, chain_tree, make_config,
                  make_workload, restrict, to_f32, uniform_tree)

__all__ = ["CONFIGS", "Workload", "bf16_bits", "bf16_to_f32", "bounded_tree", "chain_tree", "make_config",
           "make_workload", "restrict", "to_f32", "uniform_tree"]
