"""Seeded synthetic inputs for the MoE-layer workloads.

This package is shared by the tests, the benchmark and the CPU oracle's callers.
It draws random numbers and stores them in the input formats (fp32, or bf16 bit
patterns); it holds none of the layer's own arithmetic (routing, dispatch, the
expert FFN, quantisation or combine).
"""
from .gen import (CONFIGS, Workload, bf16_bits_from_f32, bf16_bits_to_f32,
                  make_workload)

__all__ = ["CONFIGS", "Workload", "make_workload", "bf16_bits_from_f32",
           "bf16_bits_to_f32"]
