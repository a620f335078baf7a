"""OCP E4M3 ("e4m3fn") codec written from the format definition (test infrastructure only).

The pages name FP8 formats but do not define the 8-bit encoding; the OCP
8-bit floating point specification (OFP8) fixes E4M3 as: 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
m * 2**-9; S.1111.111 is NaN; there are no infinities; the largest finite
magnitude is S.1111.110 = 1.75 * 2**8 = 448.

Encoding rule used here: the caller clamps to [-448, 448] first (the
quantizer does), then the value is rounded to the nearest E4M3 value, ties to
even.  The sign of the input (including -0.0) is kept in bit 7.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6
_SUB_QUANTUM = 2.0 ** -9


def e4m3_encode(v):
    """Encode binary32 values in [-448, 448] to E4M3 codes (uint8), RNE."""
    v = np.asarray(v, dtype=np.float32)
    if np.any(np.isnan(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite inputs already clamped to +-448")
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v)

    # Spacing of E4M3 values around a: 2**(E-3) with E = floor(log2 a) for
    # normals; below 2**-6 every value is a multiple of the subnormal quantum.
    _, e = np.frexp(a)                        # a = f * 2**e, f in [0.5, 1)
    E = np.maximum(e - 1, -6)
    quantum = np.ldexp(1.0, E - 3)
    q = np.rint(a / quantum)                  # a/quantum is exact (power of two); rint = half-even
    val = q * quantum                         # the rounded magnitude (exact)

    # Bit pattern of the rounded magnitude.
    _, e2 = np.frexp(val)
    E2 = e2 - 1
    normal = val >= _MIN_NORMAL
    mant = np.where(normal, val / np.ldexp(1.0, np.where(normal, E2, 0)) * 8.0 - 8.0, 0.0)
    code_norm = ((E2 + 7) << 3).astype(np.int64) + mant.astype(np.int64)
    code_sub = (val / _SUB_QUANTUM).astype(np.int64)
    code = np.where(normal, code_norm, code_sub)
    code = code | np.where(sign, 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(codes):
    """Decode E4M3 codes (uint8) to float64 values; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * _SUB_QUANTUM
    nor = (1.0 + m / 8.0) * np.ldexp(1.0, ex - 7)
    val = np.where(ex == 0, sub, nor) * s
    return np.where((ex == 0xF) & (m == 0x7), np.nan, val)
