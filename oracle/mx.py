"""MXFP8 quantized linear (E4M3 elements, one E8M0 scale per 32 values along K),
and MXFP4 weights (E2M1 elements) beside MXFP8 activations -- test
infrastructure only.

Source.  Noticias, "¿Qué son vLLM y Helion?", lists the quantized linear
formats that vLLM's linear backends serve: FP8 and INT8 (the three formats of
the rest of this package) and also INT4 and NVFP4, a block-scaled format
whose scales are applied inside the matrix product.  On gfx950 the
corresponding hardware format is OCP microscaling ("MX"): the matrix-core
instruction v_mfma_scale_f32_16x16x128_f8f6f4 multiplies each run of 32
elements by a power of two given per row.  The pages define no such format,
so the reading here is the OCP Microscaling Formats (MX) v1.0 specification,
MXFP8 with E4M3 elements:

  * a block is 32 consecutive values of one row along K (of X per token, of
    W per output channel);
  * its shared scale is X = 2**e with e = floor(log2(amax)) - 8, where amax is
    the largest magnitude in the block and 8 is the exponent of E4M3's largest
    normal (448 = 1.75 * 2**8); e is clamped to [-127, 127] and stored as the
    E8M0 byte e + 127.  An all-zero block gets e = -127 (byte 0);
  * each element is v / X rounded to the nearest E4M3 value, ties to even,
    after clamping to [-448, 448] (amax / X lies in [256, 512), so only the
    top of that range is clamped).  v / X is exact: X is a power of two.

The product of two MX operands is

    Y[m, n] = sum_b 2**(ea[m, b] + ew[n, b]) * P_b[m, n],
    P_b[m, n] = sum_{k in block b} a[m, k] * w[n, k]   (decoded E4M3 values)

with no scale epilogue: the matrix instruction applies the scales, and the
output is bf16(Y).  Exactness: every E4M3 product is a multiple of 2**-18 with
magnitude < 2**17.7, so each P_b (32 products) is exact in binary64; the
sum over blocks of P_b times a power of two is taken with ``math.fsum``,
which returns the correctly rounded binary64 value of the exact sum.

MXFP4 (the same specification, E2M1 elements: 1 sign, 2 exponent bits with
bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6): the shared
exponent is floor(log2(amax)) - 2 (6 = 1.5 * 2**2), elements are w / 2**e
clamped to +-6 and rounded to nearest E2M1, ties to even.  Here it quantizes
the weights only; the activations stay MXFP8 (the decode stream is the
weights, and 4-bit activations would cost accuracy for no bandwidth).
"""

import math

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode
from .fpbits import bf16_bits_from_f32, bf16_bits_to_f32, f32

MX_BLOCK = 32
E8M0_BIAS = 127
E4M3_EMAX = 8          # exponent of E4M3's largest normal, 448 = 1.75 * 2**8
U32 = 2.0 ** -24


def mx_shared_exponent(amax):
    """e = floor(log2(amax)) - 8, clamped to [-127, 127]; -127 where amax == 0."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)                       # a = f * 2**ex with f in [0.5, 1)
    e = (ex - 1) - E4M3_EMAX
    e = np.where(a == 0, -E8M0_BIAS, e)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def mx_quantize(x_bits):
    """Quantize bf16 rows to MXFP8.

    x_bits: uint16 [R, C] bf16 bit patterns, C % 32 == 0.
    Returns (codes uint8 [R, C] E4M3, scales uint8 [R, C/32] E8M0).
    """
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    R, C = x.shape
    if C % MX_BLOCK:
        raise ValueError("MXFP8 needs the row length to be a multiple of 32")
    blocks = x.reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2) if C else np.zeros((R, 0))
    e = mx_shared_exponent(amax)
    t = blocks * np.ldexp(1.0, -e)[:, :, None]           # exact: power-of-two scaling
    t = np.clip(t, -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(t.reshape(R, C))
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def mx_dequantize(codes, scales):
    """Real values of MXFP8 codes as float64 [R, C]."""
    c = e4m3_decode(codes)
    R, C = c.shape
    e = np.asarray(scales, dtype=np.int64) - E8M0_BIAS
    return (c.reshape(R, C // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, e)[:, :, None]).reshape(R, C)


def _block_products(a_codes, w_codes, absolute=False):
    """P_b[m, n] for every block b: float64 [nb, M, N], exact."""
    a = e4m3_decode(a_codes)
    w = e4m3_decode(w_codes)
    if absolute:
        a, w = np.abs(a), np.abs(w)
    M, K = a.shape
    nb = K // MX_BLOCK
    return np.stack([a[:, b * MX_BLOCK:(b + 1) * MX_BLOCK] @ w[:, b * MX_BLOCK:(b + 1) * MX_BLOCK].T
                     for b in range(nb)]) if nb else np.zeros((0, M, w.shape[0]))


def _scale_exponents(a_scales, w_scales):
    """ea[m, b] + ew[n, b] as int64 [nb, M, N]."""
    ea = np.asarray(a_scales, dtype=np.int64) - E8M0_BIAS
    ew = np.asarray(w_scales, dtype=np.int64) - E8M0_BIAS
    return ea.T[:, :, None] + ew.T[:, None, :]


def mx_contract_exact(a_codes, a_scales, w_codes, w_scales):
    """y_true[m, n]: the exact MX product, correctly rounded to binary64."""
    P = _block_products(a_codes, w_codes)
    E = _scale_exponents(a_scales, w_scales)
    terms = np.ldexp(P, E)                     # exact: P_b times a power of two (no overflow here)
    nb, M, N = terms.shape
    flat = terms.reshape(nb, M * N)
    return np.array([math.fsum(flat[:, i]) for i in range(M * N)], dtype=np.float64).reshape(M, N)


def mx_contract_abs(a_codes, a_scales, w_codes, w_scales):
    """sum_b 2**(ea+ew) * sum_k |a_k w_k| in float64 [M, N] (for the bound)."""
    P = _block_products(a_codes, w_codes, absolute=True)
    E = _scale_exponents(a_scales, w_scales)
    return np.sum(np.ldexp(P, E), axis=0) if P.shape[0] else np.zeros(P.shape[1:])


class MxBound:
    """The FP8 bound for an MX product, per element:

        B[m, n] = (gamma_d * sum_b 2**(ea+ew) sum_{k in b} |a_k w_k| + allowance) * (1 + 4u)

    -- binary32 sums of depth d, plus the matrix instruction's cut of small
    products (``matrix_core``), both over the products with their block
    scales applied (the scaled instruction multiplies exact products by exact
    powers of two, then adds them as the unscaled one does; the block scale
    shifts the alignment exponent).  ``fp4``: E2M1 weights.  The allowance
    is evaluated only where asked (``at``)."""

    def __init__(self, a_codes, a_scales, w_codes, w_scales, depth, matrix_core=True, fp4=False):
        from .matrix_core import e2m1_exponent, e4m3_exponent
        ea = np.asarray(a_scales, np.int64) - E8M0_BIAS
        ew = np.asarray(w_scales, np.int64) - E8M0_BIAS
        a = e4m3_decode(a_codes)
        w = e2m1_decode(w_codes) if fp4 else e4m3_decode(w_codes)
        self.av = a * np.repeat(np.ldexp(1.0, ea), MX_BLOCK, axis=1)
        self.wv = w * np.repeat(np.ldexp(1.0, ew), MX_BLOCK, axis=1)
        self.ea = (e4m3_exponent(a_codes) + np.repeat(ea, MX_BLOCK, axis=1)).astype(np.int16)
        self.ew = ((e2m1_exponent(w_codes) if fp4 else e4m3_exponent(w_codes))
                   + np.repeat(ew, MX_BLOCK, axis=1)).astype(np.int16)
        self.matrix_core = matrix_core
        gamma = depth * U32 / (1.0 - depth * U32)
        self.base = gamma * (np.abs(self.av) @ np.abs(self.wv).T) * (1.0 + 4.0 * U32)
        self.shape = self.base.shape

    def at(self, mi, ni):
        from .matrix_core import allowance_pairs
        mi, ni = np.asarray(mi, np.int64), np.asarray(ni, np.int64)
        b = self.base[mi, ni]
        if self.matrix_core and mi.size:
            b = b + allowance_pairs(self.av, self.ea, self.wv, self.ew, mi, ni).sum(axis=1) * (1.0 + 4.0 * U32)
        return b

    def full(self):
        M, N = self.shape
        mi, ni = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        return self.at(mi.reshape(-1), ni.reshape(-1)).reshape(M, N)


def mx_tolerance_bound(a_codes, a_scales, w_codes, w_scales, depth, matrix_core=True):
    """``MxBound`` for every element, float64 [M, N]."""
    return MxBound(a_codes, a_scales, w_codes, w_scales, depth, matrix_core).full()


# ----------------------------------------------------------------------------
# MXFP4 weights (OCP MX v1.0, E2M1 elements) beside MXFP8 activations.
# ----------------------------------------------------------------------------

E2M1_MAX = 6.0
E2M1_EMAX = 2          # exponent of E2M1's largest normal, 6 = 1.5 * 2**2


def e2m1_decode(codes):
    """Values of E2M1 codes (low 4 bits: sign, 2 exponent bits with bias 1,
    1 mantissa bit; exponent field 0 holds the subnormal m * 0.5)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    ex, m = (c >> 1) & 0x3, c & 0x1
    mag = np.where(ex == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, ex - 1))
    return sign * mag


def e2m1_encode(v):
    """E2M1 codes (uint8, low nibble) of values in [-6, 6], round to nearest,
    ties to even (the even code has mantissa bit 0); the sign of -0.0 kept."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)) or np.any(np.abs(v) > E2M1_MAX):
        raise ValueError("e2m1_encode expects finite inputs already clamped to +-6")
    table = e2m1_decode(np.arange(8))                  # the 8 magnitudes, increasing
    a = np.abs(v)[..., None]
    d = np.abs(a - table)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                   # one nearest value, or two at a tie
    even = (np.arange(8) & 1) == 0
    code = np.where(np.any(cand & even, axis=-1), np.argmax(cand & even, axis=-1), np.argmax(cand, axis=-1))
    return (code | np.where(np.signbit(v), 0x8, 0)).astype(np.uint8)


def mx4_shared_exponent(amax):
    """e = floor(log2(amax)) - 2, clamped to [-127, 127]; -127 where amax == 0."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)
    e = np.where(a == 0, -E8M0_BIAS, (ex - 1) - E2M1_EMAX)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def mx4_quantize(w_bits):
    """Quantize bf16 rows to MXFP4: E2M1 codes (one per element, uint8 [R, C])
    and E8M0 scales [R, C/32]; elements are w / 2**e clamped to +-6."""
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    R, C = w.shape
    if C % MX_BLOCK:
        raise ValueError("MXFP4 needs the row length to be a multiple of 32")
    blocks = w.reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2) if C else np.zeros((R, 0))
    e = mx4_shared_exponent(amax)
    t = np.clip(blocks * np.ldexp(1.0, -e)[:, :, None], -E2M1_MAX, E2M1_MAX)
    return e2m1_encode(t.reshape(R, C)), (e + E8M0_BIAS).astype(np.uint8)


def mx4_contract_exact(a_codes, a_scales, w_codes, w_scales):
    """y_true of MXFP8 activations times MXFP4 weights, correctly rounded to
    binary64: every product is a multiple of 2**-10 below 2**11.4, so each
    32-product block sum is exact, and the blocks are added with fsum."""
    a = e4m3_decode(a_codes)
    w = e2m1_decode(w_codes)
    M, K = a.shape
    nb = K // MX_BLOCK
    P = np.stack([a[:, b * MX_BLOCK:(b + 1) * MX_BLOCK] @ w[:, b * MX_BLOCK:(b + 1) * MX_BLOCK].T
                  for b in range(nb)]) if nb else np.zeros((0, M, w.shape[0]))
    terms = np.ldexp(P, _scale_exponents(a_scales, w_scales))
    flat = terms.reshape(nb, -1)
    return np.array([math.fsum(flat[:, i]) for i in range(flat.shape[1])],
                    dtype=np.float64).reshape(M, w.shape[0])


def mx4_tolerance_bound(a_codes, a_scales, w_codes, w_scales, depth, matrix_core=True):
    """The MXFP8 bound with E2M1 weight values, for every element."""
    return MxBound(a_codes, a_scales, w_codes, w_scales, depth, matrix_core, fp4=True).full()


def mx4_reference(x_bits, w_bits):
    """MXFP8 activations (mx_quantize) times MXFP4 weights (mx4_quantize)."""
    a_q, s_a = mx_quantize(x_bits)
    w_q, s_w = mx4_quantize(w_bits)
    y_true = mx4_contract_exact(a_q, s_a, w_q, s_w)
    return dict(a_q=a_q, s_a=s_a, w_q=w_q, s_w=s_w, y_true=y_true,
                y_ref=bf16_bits_from_f32(f32(y_true)))


def mx_reference(x_bits, w_bits):
    """End to end: quantize X [M, K] and W [N, K], contract exactly, round.

    Returns a dict with a_q, s_a (E8M0 bytes [M, K/32]), w_q, s_w
    ([N, K/32]), y_true (float64) and y_ref = bf16(fl(y_true)) bits."""
    a_q, s_a = mx_quantize(x_bits)
    w_q, s_w = mx_quantize(w_bits)
    y_true = mx_contract_exact(a_q, s_a, w_q, s_w)
    return dict(a_q=a_q, s_a=s_a, w_q=w_q, s_w=s_w, y_true=y_true,
                y_ref=bf16_bits_from_f32(f32(y_true)))
