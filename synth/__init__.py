"""Seeded synthetic input generators shared by the oracle tests and the GPU path."""
from .inputs import (PAGED_WORKLOADS, WORKLOADS, PagedWorkload, Workload, bf16_bits_to_f32, bf16_rne_bits,
                     make_ffn_weights, make_grad_out, make_paged_decode, make_paged_workload, make_qkv, make_workload, normal_bf16, paged_layout,
                     paged_seq_lens, stress_positions)

__all__ = ["PAGED_WORKLOADS", "WORKLOADS", "PagedWorkload", "Workload", "bf16_bits_to_f32", "bf16_rne_bits",
           "make_ffn_weights", "make_grad_out", "make_paged_decode", "make_paged_workload", "make_qkv", "make_workload", "normal_bf16",
           "paged_layout", "paged_seq_lens", "stress_positions"]
