"""Exact-arithmetic evaluation of the quantiser definitions (test helper).

Independent of the numpy oracle: values are python Fractions, fp32 rounding is
done by explicit round-half-even on the binary32 grid, and the E4M3 cast
scans the 127 non-negative finite code values with exact comparisons.  Only
for tiny inputs (it is slow).
"""

import math
import struct
from fractions import Fraction

F448 = Fraction(448)


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(b):
    return struct.unpack("<f", struct.pack("<I", b))[0]


def rn_f32(q):
    """Round a Fraction to the nearest binary32 value, ties to even (no overflow)."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def _code_value(c):
    e, m = (c >> 3) & 15, c & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(1, 64)
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


POS_VALUES = [_code_value(c) for c in range(0x7F)]


def e4m3_code(v, negative):
    """Code of the nearest E4M3 value to Fraction v (ties to even code), saturating at 448."""
    a = abs(Fraction(v))
    if a >= F448:
        code = 0x7E
    else:
        best, bestd = None, None
        for c, val in enumerate(POS_VALUES):
            d = abs(val - a)
            if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
                best, bestd = c, d
        code = best
    return code | (0x80 if negative else 0)


def quant_group(values):
    """values: fp32-representable python floats.  Returns (S as Fraction, list of codes)."""
    amax = max(abs(Fraction(x)) for x in values)
    s = Fraction(1) if amax == 0 else rn_f32(amax / F448)
    codes = [e4m3_code(rn_f32(Fraction(x) / s), math.copysign(1.0, x) < 0) for x in values]
    return s, codes


def decode(c):
    v = POS_VALUES[c & 0x7F]
    return -v if c & 0x80 else v
