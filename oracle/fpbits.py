"""Floating-point helpers for the oracle (test infrastructure only).

Conventions used throughout the oracle:
  * ``f32(x)``: one IEEE binary32 rounding, round-to-nearest-even.  numpy's
    float64 -> float32 cast is that rounding; float32 array arithmetic in numpy
    (``*``, ``/``) is one IEEE binary32 operation per element, also RNE.
  * bf16 values are carried as their uint16 bit patterns so that comparisons
    are bit comparisons.

The pages fix no rounding mode; round-to-nearest-even everywhere is the plain
reading (IEEE default).  These helpers are pinned against an exact rational
rounding routine written separately in the tests.
"""

import numpy as np


def f32(x):
    """Round values (float64 or integer, magnitude < 2**53) to binary32, RNE."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits_from_f32(x):
    """Round binary32 values to bfloat16 (RNE); return the uint16 bit patterns.

    bfloat16 keeps the top 16 bits of binary32.  Round-to-nearest-even on the
    discarded 16 bits: add 0x7FFF plus the lowest kept bit, then truncate.
    Overflow past the largest finite bf16 carries into the exponent and gives
    infinity, which is the RNE result.  NaN stays a quiet NaN of the same sign.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        r = r.copy()
        r[nan] = ((u[nan] >> 16).astype(np.uint16) | 0x0040)
    return r


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def ulp_bf16(bits):
    """One unit in the last place of the bf16 value(s) given as bit patterns.

    For a normal bf16 value with |y| in [2**e, 2**(e+1)) the spacing is
    2**(e-7) (8 significand bits).  Zero and subnormals share the subnormal
    spacing 2**-133.  Returned as float64.
    """
    y = np.abs(bf16_bits_to_f32(bits).astype(np.float64))
    _, e = np.frexp(y)            # y = f * 2**e, f in [0.5, 1)
    ulp = np.ldexp(1.0, e - 8)     # floor(log2 y) = e - 1; spacing 2**(e-1-7)
    tiny = y < 2.0 ** -126
    return np.where(tiny, 2.0 ** -133, ulp)
