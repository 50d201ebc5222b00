"""OCP E4M3FN codec (oracle; test infrastructure only).

The pages (paper.rainbus.top, section "FP8 量化 (E4M3 格式)") fix the format as
4 exponent bits plus 3 mantissa bits with largest representable magnitude 448,
and write the quantiser as X_hat = [X / S_X] with S_X = max|X| / 448.  The
bracket is read as a cast to the nearest representable E4M3 value, ties to the
even code, saturating at 448; the sign of zero is kept.

Format (OCP 8-bit floating point, E4M3FN): bias 7, no infinities, code 0x7F and
0xFF are NaN; exponent field e = 1..15 gives (1 + m/8) * 2**(e-7), e = 0 gives
the subnormals (m/8) * 2**-6.  Largest finite code 0x7E = 448.

The encoder is deliberately the slow, obviously correct form: find the two
neighbouring table entries and pick the nearer one.
"""

import numpy as np

E4M3_MAX = 448.0


def _decode_code(c):
    """Value of one E4M3FN code (python float, exact)."""
    sign = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)
# non-negative finite values in code order 0x00..0x7E; they ascend with the code
_POS = _TABLE[:0x7F].copy()


def e4m3_table():
    """All 256 code values as float64 (NaN for 0x7F and 0xFF)."""
    return _TABLE.copy()


def e4m3_decode(q):
    """Decode uint8 codes to float64 values (exact)."""
    q = np.asarray(q, dtype=np.uint8)
    return _TABLE[q]


def e4m3_encode(f):
    """Cast float32 values to E4M3FN codes: nearest, ties to even code, saturating.

    ``f`` must be finite.  |f| >= 448 gives the largest finite code (the band
    [448, 464) rounds to 448 anyway, 464 ties to 448, and anything larger would
    round to 480, which does not exist).  Returns uint8 codes with the sign bit
    copied from ``f`` (so -0.0 gives 0x80).
    """
    f = np.asarray(f, dtype=np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("e4m3_encode: non-finite input is outside the contract")
    a = np.abs(f).astype(np.float64)  # exact widening
    lo_idx = np.searchsorted(_POS, a, side="right") - 1  # _POS[lo_idx] <= a
    lo_idx = np.clip(lo_idx, 0, 0x7E)
    hi_idx = np.minimum(lo_idx + 1, 0x7E)
    lo = _POS[lo_idx]
    hi = _POS[hi_idx]
    d_lo = a - lo  # exact in float64: both operands have <= 24 significant bits
    d_hi = hi - a
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    # on a tie take whichever neighbour has the even code
    pick_hi = np.where(tie, (hi_idx % 2) == 0, pick_hi)
    code = np.where(pick_hi, hi_idx, lo_idx)
    code = np.where(a >= E4M3_MAX, 0x7E, code).astype(np.uint8)
    sign = np.signbit(f).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)
