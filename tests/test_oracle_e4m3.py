"""Pins of the oracle's E4M3 codec (no GPU).

The format is fixed by the Jet-RL pages (paper.rainbus.top, section
"FP8 量化 (E4M3 格式)": 4 exponent bits, 3 mantissa bits, largest value 448) and
the OCP E4M3FN definition; the cast is read as nearest, ties to even code,
saturating.  Pins: closed-form table facts, hand-derived golden cases, an
independent bit-arithmetic encoder, exact Fraction arithmetic, and torch's
float8_e4m3fn cast (library) where it agrees by definition (|x| <= 448).
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import exact
import golden_io
from oracle import e4m3_decode, e4m3_encode, e4m3_table

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_table_closed_form():
    t = e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x78] == 256.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 00..7e must ascend"
    assert np.array_equal(t[0x80:0xFF], -pos)
    # 126 positive finite nonzero values, spacing doubles each binade
    assert np.count_nonzero(pos > 0) == 126
    for e in range(1, 16):
        binade = pos[8 * e: 8 * e + 8]
        assert np.all(np.diff(binade) == 2.0 ** (e - 7) / 8)


def test_decode_matches_exact():
    t = e4m3_table()
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert Fraction(t[c]) == exact.decode(c)
        assert e4m3_decode(np.array([c], np.uint8))[0] == t[c]


def test_golden_cases():
    cases = golden_io.e4m3_cases()
    x = np.array([v for v, _ in cases], np.float32)
    got = e4m3_encode(x)
    want = np.array([c for _, c in cases], np.uint8)
    bad = [(v, hex(g), hex(w)) for v, g, w in zip(x, got, want) if g != w]
    assert not bad, bad


def bitwise_encode(f):
    """Independent encoder: integer arithmetic on the binary32 bit pattern."""
    f = np.asarray(f, np.float32)
    b = f.view(np.uint32).astype(np.int64)
    sign = (b >> 24) & 0x80
    a = b & 0x7FFFFFFF
    out = np.zeros_like(a)
    sat = a >= 0x43E00000  # |f| >= 448
    sub = a < 0x3C800000   # |f| < 2^-6
    # normal: round the 23-bit mantissa to 3 bits, nearest even, then rebias 127 -> 7
    r = a + 0x7FFFF + ((a >> 20) & 1)
    out = np.where(~sat & ~sub, (r >> 20) - (120 << 3), out)
    # subnormal: multiple of 2^-9, nearest even integer
    t = np.abs(f.astype(np.float64)) * 512.0
    fl = np.floor(t)
    rem = t - fl
    n = fl + ((rem > 0.5) | ((rem == 0.5) & (fl % 2 == 1)))
    out = np.where(sub, n.astype(np.int64), out)
    out = np.where(sat, 0x7E, out)
    return (out | sign).astype(np.uint8)


def _boundary_set():
    """Every E4M3 value and midpoint, with the 8 fp32 neighbours on each side."""
    pos = e4m3_table()[:0x7F]
    pts = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2, [464.0, 480.0, 512.0]]).astype(np.float32)
    b = pts.view(np.uint32).astype(np.int64)
    nb = (b[:, None] + np.arange(-8, 9)[None, :]).ravel()
    nb = nb[(nb >= 0) & (nb < 0x7F800000)].astype(np.uint32)
    v = nb.view(np.float32)
    return np.concatenate([v, -v])


def _test_sets():
    rng = np.random.default_rng(12345)
    all_bf16 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    all_bf16 = all_bf16[np.isfinite(all_bf16)]
    strided = (np.arange(0, 0x44800000, 1021, dtype=np.uint32)).view(np.float32)  # [0, 1024)
    rnd = rng.integers(0, 0x7F800000, size=400000, dtype=np.uint32).view(np.float32)
    subn = np.arange(0, 1 << 16, dtype=np.uint32).view(np.float32)  # fp32 subnormals
    return {"bf16": all_bf16, "boundary": _boundary_set(), "strided": np.concatenate([strided, -strided]),
            "random": np.concatenate([rnd, -rnd]), "subnormal": np.concatenate([subn, -subn])}


@pytest.mark.parametrize("name", ["bf16", "boundary", "strided", "random", "subnormal"])
def test_against_bitwise_encoder(name):
    x = _test_sets()[name]
    got, want = e4m3_encode(x), bitwise_encode(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("name", ["bf16", "boundary", "strided", "random", "subnormal"])
def test_against_torch_float8(name):
    x = _test_sets()[name]
    x = x[np.abs(x) <= 448.0]  # torch's cast does not saturate above 448 (gives NaN)
    want = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3_encode(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_against_exact_fractions():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(300).astype(np.float32) * np.float32(50),
        rng.standard_normal(300).astype(np.float32) * np.float32(0.01),
        _boundary_set()[::37],
    ]).astype(np.float32)
    got = e4m3_encode(x)
    for v, g in zip(x, got):
        assert g == exact.e4m3_code(Fraction(float(v)), math.copysign(1.0, float(v)) < 0), v


def test_roundtrip_and_saturation():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes).astype(np.float32)), codes)
    big = np.array([448.0, 449.0, 464.0, 465.0, 1e30, -3e38], np.float32)
    assert np.array_equal(e4m3_encode(big), np.array([0x7E] * 5 + [0xFE], np.uint8))
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.nan], np.float32))
