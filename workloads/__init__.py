"""Seeded synthetic inputs shared by the CPU oracle's tests and the GPU path."""
from .synth import (GATE_SIGMOID, GATE_SOFTMAX, WORKLOADS, Workload, bf16_bits_to_f32,
                    custom, f32_to_bf16_bits, make, output_grad)

__all__ = ["GATE_SIGMOID", "GATE_SOFTMAX", "WORKLOADS", "Workload", "bf16_bits_to_f32",
           "custom", "f32_to_bf16_bits", "make", "output_grad"]
