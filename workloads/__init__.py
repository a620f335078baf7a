"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This package holds no arithmetic of the method (no quantization, no
contraction): only the shapes of the workloads and the seeded random draws
of bf16 activations and weights.  Both the CPU oracle and the GPU path take
their inputs from here.
"""

from .configs import CONFIGS, Workload, decode_points, config_by_name
from .synth import make_inputs, bf16_bits

__all__ = ["CONFIGS", "Workload", "decode_points", "config_by_name", "make_inputs", "bf16_bits"]
