"""An exact-rational restatement of the quantized linear, for pinning the oracle.

Written separately from ``oracle/``: Python ``Fraction`` arithmetic, its own
generic round-to-nearest-even float rounding, its own E4M3 value table built
from the OCP OFP8 format definition, and integer / rational sums.  It is far
too slow for anything but tiny inputs, which is all it is for.
"""

from fractions import Fraction as F


def round_float(x, mant_bits, emin):
    """Round the rational x to the nearest binary float, ties to even.

    mant_bits: significand bits including the implicit one (24 for binary32,
    8 for bfloat16, 4 for E4M3); emin: exponent of the smallest normal.
    Gradual underflow (subnormals) is modelled; overflow is not needed here.
    """
    if x == 0:
        return F(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = F(2) ** (e - (mant_bits - 1))
    q = a / quantum
    n = q.numerator // q.denominator
    r = q - n
    if r > F(1, 2) or (r == F(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * quantum


def r32(x):
    return round_float(F(x), 24, -126)


def rbf16(x):
    return round_float(F(x), 8, -126)


def re4m3(x):
    return round_float(F(x), 4, -6)


def e4m3_value_table():
    """code -> Fraction value (None for NaN), from the OFP8 E4M3 definition."""
    tab = {}
    for c in range(256):
        s = -1 if c & 0x80 else 1
        ex, m = (c >> 3) & 0xF, c & 7
        if ex == 0xF and m == 7:
            tab[c] = None
        elif ex == 0:
            tab[c] = s * F(m, 512)
        else:
            tab[c] = s * (1 + F(m, 8)) * F(2) ** (ex - 7)
    return tab


E4M3 = e4m3_value_table()


def rint_even(q):
    n = q.numerator // q.denominator
    r = q - n
    if r > F(1, 2) or (r == F(1, 2) and n % 2 == 1):
        n += 1
    return n


def quantize_group(values, negzero, Q, kind):
    """values: list of Fractions (bf16 inputs); negzero: list of bools (input is -0.0).

    Returns (codes, s) where codes are ints (int8 values) or (value, sign) pairs for E4M3.
    """
    amax = max((abs(v) for v in values), default=F(0))
    s = F(1) if amax == 0 else r32(amax / Q)
    out = []
    for v, nz in zip(values, negzero):
        t = r32(v / s)
        if kind == "int8":
            out.append(max(-127, min(127, rint_even(t))))
        else:
            t = max(F(-448), min(F(448), t))
            val = re4m3(t)
            neg = v < 0 or (v == 0 and nz)
            out.append((val, neg))
    return out, s


def dot_int(a_row, w_row):
    return sum(int(x) * int(y) for x, y in zip(a_row, w_row))


def dot_frac(a_row, w_row):
    return sum((x * y for x, y in zip(a_row, w_row)), F(0))


def floor_log2(a):
    """floor(log2 a) of a positive rational, by integer comparison."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    return e


def mx_quantize_block(values, negzero):
    """One MXFP8 block (OCP MX: shared exponent floor(log2 amax) - 8, clamped to
    [-127, 127]; -127 for an all-zero block; elements v / 2**e clamped to
    +-448 and rounded to E4M3).  Returns ([(value, neg)], e)."""
    amax = max((abs(v) for v in values), default=F(0))
    e = -127 if amax == 0 else max(-127, min(127, floor_log2(amax) - 8))
    out = []
    for v, nz in zip(values, negzero):
        t = max(F(-448), min(F(448), v / F(2) ** e))
        out.append((re4m3(t), v < 0 or (v == 0 and nz)))
    return out, e


def re2m1(x):
    """Round to E2M1 (2 significand bits, smallest normal exponent 0, so the
    subnormal quantum is 1/2), ties to even."""
    return round_float(F(x), 2, 0)


def mx4_quantize_block(values, negzero):
    """One MXFP4 block: e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for
    an all-zero block); elements v / 2**e clamped to +-6, rounded to E2M1."""
    amax = max((abs(v) for v in values), default=F(0))
    e = -127 if amax == 0 else max(-127, min(127, floor_log2(amax) - 2))
    out = []
    for v, nz in zip(values, negzero):
        t = max(F(-6), min(F(6), v / F(2) ** e))
        out.append((re2m1(t), v < 0 or (v == 0 and nz)))
    return out, e
