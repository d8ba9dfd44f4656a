"""Seeded synthetic input generators shared by the oracle tests and the GPU path."""
from .inputs import (WORKLOADS, Workload, bf16_bits_to_f32, bf16_rne_bits, make_qkv,
                     make_workload, normal_bf16, stress_positions)

__all__ = ["WORKLOADS", "Workload", "bf16_bits_to_f32", "bf16_rne_bits", "make_qkv",
           "make_workload", "normal_bf16", "stress_positions"]
