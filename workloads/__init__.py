"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This package holds no arithmetic of the method (no quantization, no
contraction): only the shapes of the workloads and the seeded random draws
of bf16 activations and weights.  Both the CPU oracle and the GPU path take
their inputs from here.
"""

from .configs import CONFIGS, Workload, config_by_name, decode_points, decode_workloads
from .synth import make_inputs, bf16_bits

__all__ = ["CONFIGS", "Workload", "config_by_name", "decode_points", "decode_workloads", "make_inputs", "bf16_bits"]
