"""Exact-arithmetic evaluation of the quantiser definitions (test helper).

Independent of the numpy oracle: values are python Fractions, fp32 rounding is
done by explicit round-half-even on the binary32 grid, and the E4M3 cast
scans the 127 non-negative finite code values with exact comparisons.  Only
for tiny inputs (it is slow).
"""

import bisect
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
assert all(a < b for a, b in zip(POS_VALUES, POS_VALUES[1:]))


def e4m3_code(v, negative):
    """Code of the nearest E4M3 value to Fraction v (ties to even code), saturating at 448."""
    a = abs(Fraction(v))
    if a >= F448:
        code = 0x7E
    else:
        # POS_VALUES increases with the code: compare with the two neighbours
        hi = bisect.bisect_left(POS_VALUES, a)
        if POS_VALUES[hi] == a:
            code = hi
        else:
            lo = hi - 1
            dl, dh = a - POS_VALUES[lo], POS_VALUES[hi] - a
            code = lo if dl < dh or (dl == dh and lo % 2 == 0) else hi
    return code | (0x80 if negative else 0)


def quant_group(values):
    """values: fp32-representable python floats.  Returns (S as Fraction, list of codes)."""
    amax = max(abs(Fraction(x)) for x in values)
    s = rn_f32(amax / F448)
    if s == 0:  # amax == 0, or amax / 448 below half the smallest fp32 subnormal
        s = Fraction(1)
    codes = [e4m3_code(rn_f32(Fraction(x) / s), math.copysign(1.0, x) < 0) for x in values]
    return s, codes


def decode(c):
    v = POS_VALUES[c & 0x7F]
    return -v if c & 0x80 else v


def _pow2_floor_exp(a):
    """e with 2^e <= a < 2^(e+1) for a positive Fraction a."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    return e


def rn_sqrt_f32(d):
    """The binary32 value nearest to sqrt(d) (ties to even) for a Fraction d >= 0
    whose square root lies in the normal fp32 range."""
    d = Fraction(d)
    if d == 0:
        return Fraction(0)
    # sqrt(d) in [2^e, 2^(e+1)) with e = floor(log2(d) / 2)
    e = _pow2_floor_exp(d) // 2
    quantum = Fraction(2) ** (e - 23)
    a = d / (quantum * quantum)          # sqrt(a) = sqrt(d) / quantum, in [2^23, 2^24)
    fl = math.isqrt(a.numerator // a.denominator)  # floor(sqrt(a)) = isqrt(floor(a))
    half = Fraction(2 * fl + 1, 2)
    if a > half * half or (a == half * half and fl % 2 == 1):
        fl += 1
    return fl * quantum


def pairwise_tree_sum_f32(values):
    """Canonical pairwise tree over the list: adjacent pairs added level by level
    (each sum rounded to fp32), an odd last element carried up unchanged."""
    v = list(values)
    if not v:
        return Fraction(0)
    while len(v) > 1:
        nxt = [rn_f32(v[i] + v[i + 1]) for i in range(0, len(v) - 1, 2)]
        if len(v) % 2:
            nxt.append(v[-1])
        v = nxt
    return v[0]


def rmsnorm_row_exact(xs, gammas, eps):
    """The fused RMSNorm + 1x128 quantiser on one row, every fp32 step rounded
    explicitly: sq = fl32(x*x); ss = pairwise tree; ms = fl32(ss / K);
    d = fl32(ms + fl32(eps)); r = fl32(sqrt(d)); inv = fl32(1 / r);
    y = fl32(fl32(x * inv) * gamma); then quant_group on every 128 values of y.

    xs, gammas: python floats (bf16 values).  Returns (inv, [(S, codes)] per group)."""
    k = len(xs)
    xf = [Fraction(x) for x in xs]
    gf = [Fraction(g) for g in gammas]
    ss = pairwise_tree_sum_f32([rn_f32(x * x) for x in xf])
    ms = rn_f32(ss / k)
    d = rn_f32(ms + rn_f32(Fraction(eps)))
    inv = rn_f32(1 / rn_sqrt_f32(d))
    out = []
    for g0 in range(0, k, 128):
        ys, neg = [], []
        for i in range(g0, g0 + 128):
            ys.append(rn_f32(rn_f32(xf[i] * inv) * gf[i]))
            # inv > 0: the sign of y (zero included) is sign(x) xor sign(gamma)
            neg.append((math.copysign(1.0, xs[i]) < 0) != (math.copysign(1.0, gammas[i]) < 0))
        out.append(quant_group_signed(ys, neg))
    return inv, out


def quant_group_signed(values, negative):
    """quant_group for Fraction values with explicit signs (zeros keep theirs)."""
    amax = max(abs(v) for v in values)
    s = rn_f32(amax / F448)
    if s == 0:
        s = Fraction(1)
    codes = [e4m3_code(rn_f32(v / s), n) for v, n in zip(values, negative)]
    return s, codes
