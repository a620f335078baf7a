"""CPU oracle for the scaled quantized linear -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct CPU statement of what the
GPU path computes:

    Y[M,N] = s_a[m] * s_w[n] * (A_q[M,K] . W_q[N,K]^T)      (bf16 output)

plus the dynamic activation quantizer and the offline weight quantizer, for
the three formats of the pages (FP8_Dynamic, W8A8_INT8, Block_FP8), and the
SiLU-and-mul epilogue of a merged gate/up projection (``glu``), and the
MXFP8 linear (E4M3 elements with E8M0 scales per 32 values along K, the
scales applied inside the product) and its MXFP4-weight variant (``mx``).

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and nothing
here imports the product path: the two share no code.  Only the seeded input
generator in ``workloads/`` serves both sides.

Sources.  The pages are five web pages about the article "Building a
High-Performance and Portable vLLM Linear Backend with Helion" (PyTorch blog):
  * "Summary"  -- the English summary at yuxiaoba.github.io/tech/en/helion-linear/
  * "Noticias" -- the Spanish rendering "Helion entra al backend lineal de vLLM
                  y supera a CUTLASS en Hopper" (noticias.mechatronicstore.cl)
  * "News"     -- "Helion Integration Boosts vLLM Inference Speed" (latestnews.news)
Each function cites the page and section it follows.  Where the pages are
silent (the scale formula, rounding modes, layouts, op order) the reading
taken is stated in the docstring.

Pins.  Every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself: an independent exact-rational (Fraction)
implementation on tiny inputs, closed forms, layout one-hot probes, the OCP
OFP8 specification's E4M3 values, torch's CPU float8 cast, the bf16 bit
fields (MX shared exponents, exhaustively), and invariants of the method (variant order independence, quantizer bounds).  The
FP8 tolerance's matrix-core allowance (``matrix_core``) is pinned against a
brute-force restatement of its model and, on the GPU, against the matrix
instruction itself on adversarial operands.  No function is "parity
unpinned".
"""

from .fpbits import (bf16_bits_from_f32, bf16_bits_to_f32, ulp_bf16, f32)
from .e4m3 import e4m3_encode, e4m3_decode, E4M3_MAX
from .quant import (FMT_FP8_DYNAMIC, FMT_W8A8_INT8, FMT_BLOCK_FP8, FORMATS,
                    qmax_of, quantize_act, quantize_weight, dequant_codes)
from .linear import (contract_exact, contract_abs, epilogue, reference, Fp8Bound, accumulator_bound,
                     tolerance_bound, summation_depth, check_fp8_parity, parity_statistics,
                     contract_split_order, contract_swap_ab,
                     emulate_fp32_accumulation)
from .glu import silu, glu_values, glu_reference, SILU_SLOPE_MAX
from .matrix_core import allowance_pairs, allowance_full, e4m3_exponent, e2m1_exponent
from .mx import (MxBound, MX_BLOCK, mx_shared_exponent, mx_quantize, mx_dequantize, mx_contract_exact,
                 mx_contract_abs, mx_tolerance_bound, mx_reference, e2m1_encode, e2m1_decode,
                 mx4_shared_exponent, mx4_quantize, mx4_contract_exact, mx4_tolerance_bound, mx4_reference)

__all__ = [
    "bf16_bits_from_f32", "bf16_bits_to_f32", "ulp_bf16", "f32",
    "e4m3_encode", "e4m3_decode", "E4M3_MAX",
    "FMT_FP8_DYNAMIC", "FMT_W8A8_INT8", "FMT_BLOCK_FP8", "FORMATS",
    "qmax_of", "quantize_act", "quantize_weight", "dequant_codes",
    "contract_exact", "contract_abs", "epilogue", "reference",
    "tolerance_bound", "summation_depth", "Fp8Bound", "accumulator_bound", "check_fp8_parity",
    "parity_statistics", "allowance_pairs", "allowance_full", "e4m3_exponent", "e2m1_exponent", "MxBound",
    "silu", "glu_values", "glu_reference", "SILU_SLOPE_MAX",
    "contract_split_order", "contract_swap_ab", "emulate_fp32_accumulation",
    "MX_BLOCK", "mx_shared_exponent", "mx_quantize", "mx_dequantize", "mx_contract_exact",
    "mx_contract_abs", "mx_tolerance_bound", "mx_reference", "e2m1_encode", "e2m1_decode",
    "mx4_shared_exponent", "mx4_quantize", "mx4_contract_exact", "mx4_tolerance_bound", "mx4_reference",
]
