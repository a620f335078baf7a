"""SiLU-and-mul epilogue of a merged gate/up projection (test infrastructure only).

The step that follows the gate_up linear of a gated MLP: the linear's N
output columns are two halves, gate G = columns [0, I) and up U = columns
[I, 2I) (I = N/2, the merged gate-then-up row order of the projection's
weight), and the down projection consumes

    H[m, i] = silu(G[m, i]) * U[m, i],    silu(g) = g / (1 + exp(-g)).

Source: the deep-dive page ("Optimizing vLLM Linear Backend Performance
using Helion Kernel DSL", "Understanding Helion", its list of core design
principles) names activations such as SiLU as epilogues fused into the
GEMM's write-back, applied to the accumulator before the output is stored.
Reading taken here: G and U are the linear's binary32 epilogue values
(after the scales, before any bf16 rounding); H is rounded to bfloat16
once.  The page's example applies SiLU alone; feeding a down projection
takes the gated form above, of which SiLU alone is the U = 1 case.

Exactness: for INT8 the binary32 epilogue value t = fl(fl(f32(acc) s_a) s_w)
is exact, so only the binary32 evaluation of silu and the product differ
from the float64 value.  For the FP8 formats G and U carry the accumulation
bound B of the linear; it propagates through |d silu/dg| <= 1.1 and the
product.
"""

import numpy as np

from .fpbits import bf16_bits_from_f32, f32
from .linear import summation_depth, tolerance_bound

# |silu'(g)| = |s(g) (1 + g (1 - s(g)))| with s the logistic function; its
# supremum over the reals is 1.0998 (at g ~ 2.4).
SILU_SLOPE_MAX = 1.1
# binary32 evaluation of g / (1 + exp(-g)) * u: exp, add, divide, multiply,
# a few ulps of binary32 in all.
GLU_EVAL_REL = 2.0 ** -20


def silu(x):
    """x / (1 + exp(-x)) in float64 (exp overflowing to inf gives a signed 0)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def _split(t):
    t = np.asarray(t)
    if t.shape[1] % 2:
        raise ValueError("the merged gate/up output needs an even number of columns")
    half = t.shape[1] // 2
    return t[:, :half], t[:, half:]


def glu_values(t):
    """H = silu(G) * U in float64 from the merged [M, 2I] values t."""
    g, u = _split(np.asarray(t, dtype=np.float64))
    return silu(g) * u


def glu_reference(fmt, r, split=1, waves_k=16):
    """Reference and bound for the fused SiLU-and-mul output of the linear in
    ``r`` (a dict from ``reference`` over the merged [M, 2I] weight).

    Returns (h_ref bf16 bits, h_true float64, bound float64), to be checked
    with ``check_fp8_parity``: an element passes within one bf16 ulp of h_ref
    or within half a bf16 ulp plus ``bound`` of h_true."""
    from .quant import FMT_W8A8_INT8, FMT_BLOCK_FP8
    S = np.asarray(r["S"])
    if fmt == FMT_W8A8_INT8:
        sa = np.asarray(r["s_a"], np.float32)[:, None]
        sw = np.asarray(r["s_w"], np.float32)[None, :]
        t = (f32(S) * sa) * sw                      # the kernel's binary32 epilogue value, exactly
        B = np.zeros(t.shape)
    else:
        t = np.asarray(r["y_true"], dtype=np.float64)
        K = r["a_q"].shape[1]
        d = summation_depth(K, split=split, waves_k=waves_k)
        B = tolerance_bound(fmt, r["a_q"], r["w_q"], r["s_a"], r["s_w"], d)
    g, u = _split(np.asarray(t, dtype=np.float64))
    bg, bu = _split(B)
    h_true = silu(g) * u
    bound = (SILU_SLOPE_MAX * bg * (np.abs(u) + bu) + np.abs(silu(g)) * bu) * (1 + 2.0 ** -20) \
        + GLU_EVAL_REL * np.abs(h_true)
    h_ref = bf16_bits_from_f32(f32(h_true))
    return h_ref, h_true, bound
