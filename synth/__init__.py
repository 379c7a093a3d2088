"""Seeded synthetic inputs shared by the CPU oracle's tests and the HIP path."""
from .workloads import (WORKLOADS, ORDER, Workload, generate, sample_rows, random_inputs,
                        round_bf16, bf16_bits)

__all__ = ["WORKLOADS", "ORDER", "Workload", "generate", "sample_rows", "random_inputs",
           "round_bf16", "bf16_bits"]
