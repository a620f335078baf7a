"""Seeded synthetic inputs with the shape and distribution of LLM decode linears.

The pages measure on Qwen3 dense models (Summary, "Preserve the conditions
when moving from kernels to serving"); their checkpoints are not available, so
random tensors stand in for them:

  1. A ~ N(0, 1) float32 [M_max, K];
  2. outlier channels: the first n_out = max(1, round(0.01 K)) entries of a
     random permutation of K are scaled by 20 in every token (LLM activations
     carry a few large channels);
  3. W ~ N(0, sigma) float32 [N, K];
  4. both cast to bf16 (round to nearest even, torch's cast).

One torch CPU generator, seeded once per (workload, shape), draws in exactly
this order; smaller M use the first M rows of A so an M sweep shares tokens.
"""

import numpy as np
import torch


def make_inputs(K, N, M_max, sigma_w, seed=0, with_weight=True):
    """Return (x_bf16 [M_max, K], w_bf16 [N, K] or None) as CPU torch tensors."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    a = torch.randn(M_max, K, generator=g, dtype=torch.float32)
    n_out = max(1, int(round(0.01 * K))) if K > 0 else 0
    if n_out:
        idx = torch.randperm(K, generator=g)[:n_out]
        a[:, idx] *= 20.0
    x = a.to(torch.bfloat16)
    w = None
    if with_weight:
        w = (torch.randn(N, K, generator=g, dtype=torch.float32) * sigma_w).to(torch.bfloat16)
    return x, w


def bf16_bits(t):
    """uint16 numpy view of a CPU bf16 tensor's bit patterns (no copy of values)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
