"""Seeded synthetic MSA workloads (inputs only; no attention arithmetic)."""
from .gen import Workload, make_workload, random_small_case, f32_to_bf16_bits, NAMES, SMALL

__all__ = ["Workload", "make_workload", "random_small_case", "f32_to_bf16_bits", "NAMES", "SMALL"]
