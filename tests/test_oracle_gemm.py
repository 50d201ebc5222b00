"""Pins of the oracle's block-scaled GEMM references and acceptance check (no GPU).

Definitions: paper.rainbus.top, sections "GEMM 量化布局" (FProp Y = X W^T,
WGrad dW = dY^T X, DGrad dX = dY W) and "核心方法" ((1x128)x(128x128) for FProp
and DGrad, (1x128)x(128x1) for WGrad).  Pins: exact Fraction brute force on
tiny shapes, an exact-integer case with distinct power-of-two scales per
(row, block) -- any mis-indexed scale changes the result -- , DGrad against
FProp on the explicitly transposed weight, linearity, and the tolerance
function against hand-made perturbations and torch's bf16 rounding.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import exact
import oracle

CODES_SMALL = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0, 0x30], np.uint8)  # 0, +-1, +-2, 0.5


def rand_codes(rng, shape, small=False):
    if small:
        return CODES_SMALL[rng.integers(0, len(CODES_SMALL), size=shape)]
    q = rng.integers(0, 256, size=shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    return q


def pow2_scales(rng, shape, lo=-6, hi=6):
    return np.exp2(rng.integers(lo, hi, size=shape)).astype(np.float32)


def exact_fprop(qx, sx, qw, sw):
    M, K = qx.shape
    N = qw.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for kb in range(K // 128):
                p = sum(exact.decode(int(qx[m, k])) * exact.decode(int(qw[n, k]))
                        for k in range(128 * kb, 128 * kb + 128))
                acc += Fraction(float(sx[kb, m])) * Fraction(float(sw[n // 128, kb])) * p
            out[m][n] = acc
    return out


def test_fprop_exact_integer_case():
    rng = np.random.default_rng(0)
    M, N, K = 5, 256, 256
    qx, qw = rand_codes(rng, (M, K), small=True), rand_codes(rng, (N, K), small=True)
    sx = pow2_scales(rng, (K // 128, M))
    sw = pow2_scales(rng, (N // 128, K // 128))
    ref = oracle.gemm_fprop_ref(qx, sx, qw, sw)
    ex = exact_fprop(qx, sx, qw, sw)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(ref[m, n])) == ex[m][n]  # zero tolerance
    # a transposed scale layout gives a different answer (the pin has teeth)
    wrong = (oracle.dequant_groups(qx, sx.T.reshape(K // 128, M) if M == K // 128 else sx[::-1])
             @ oracle.dequant_blocks(qw, sw).T)
    assert not np.array_equal(wrong, ref)


def test_fprop_against_exact_random_codes():
    rng = np.random.default_rng(1)
    M, N, K = 3, 128, 384
    qx, qw = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sx = rng.uniform(0.001, 2.0, size=(K // 128, M)).astype(np.float32)
    sw = rng.uniform(0.0001, 0.01, size=(N // 128, K // 128)).astype(np.float32)
    ref = oracle.gemm_fprop_ref(qx, sx, qw, sw)
    ex = exact_fprop(qx, sx, qw, sw)
    for m in range(M):
        for n in range(0, N, 7):
            assert abs(Fraction(float(ref[m, n])) - ex[m][n]) <= abs(ex[m][n]) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 60)


def test_dgrad_is_fprop_on_transposed_weight():
    rng = np.random.default_rng(2)
    M, N, K = 7, 256, 384  # dY [M, N], W [N, K]
    qdy, qw = rand_codes(rng, (M, N)), rand_codes(rng, (N, K))
    sdy = rng.uniform(0.01, 1, size=(N // 128, M)).astype(np.float32)
    sw = rng.uniform(0.01, 1, size=(N // 128, K // 128)).astype(np.float32)
    d = oracle.gemm_dgrad_ref(qdy, sdy, qw, sw)
    f = oracle.gemm_fprop_ref(qdy, sdy, np.ascontiguousarray(qw.T), np.ascontiguousarray(sw.T))
    assert d.shape == (M, K)
    assert np.allclose(d, f, rtol=1e-13, atol=1e-300)


def test_dgrad_exact_integer_case():
    rng = np.random.default_rng(3)
    M, N, K = 3, 256, 256
    qdy, qw = rand_codes(rng, (M, N), small=True), rand_codes(rng, (N, K), small=True)
    sdy = pow2_scales(rng, (N // 128, M))
    sw = pow2_scales(rng, (N // 128, K // 128))
    ref = oracle.gemm_dgrad_ref(qdy, sdy, qw, sw)
    for m in range(M):
        for k in range(0, K, 5):
            acc = Fraction(0)
            for nb in range(N // 128):
                p = sum(exact.decode(int(qdy[m, n])) * exact.decode(int(qw[n, k]))
                        for n in range(128 * nb, 128 * nb + 128))
                acc += Fraction(float(sdy[nb, m])) * Fraction(float(sw[nb, k // 128])) * p
            assert Fraction(float(ref[m, k])) == acc


def test_wgrad_exact_integer_case():
    rng = np.random.default_rng(4)
    M, N, K = 256, 128, 256  # tokens, out features, in features
    qdyt, qxt = rand_codes(rng, (N, M), small=True), rand_codes(rng, (K, M), small=True)
    sdyt, sxt = pow2_scales(rng, (M // 128, N)), pow2_scales(rng, (M // 128, K))
    ref = oracle.gemm_wgrad_ref(qdyt, sdyt, qxt, sxt)
    assert ref.shape == (N, K)
    for n in range(0, N, 9):
        for k in range(0, K, 11):
            acc = Fraction(0)
            for mb in range(M // 128):
                p = sum(exact.decode(int(qdyt[n, m])) * exact.decode(int(qxt[k, m]))
                        for m in range(128 * mb, 128 * mb + 128))
                acc += Fraction(float(sdyt[mb, n])) * Fraction(float(sxt[mb, k])) * p
            assert Fraction(float(ref[n, k])) == acc


def test_sampled_references_match_full():
    rng = np.random.default_rng(5)
    M, N, K = 130, 256, 384
    qx, qw = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sx = rng.uniform(0.01, 1, size=(K // 128, M)).astype(np.float32)
    sw = rng.uniform(0.01, 1, size=(N // 128, K // 128)).astype(np.float32)
    rows, cols = np.array([0, 5, 129]), np.array([1, 128, 255])
    full = oracle.gemm_fprop_ref(qx, sx, qw, sw)
    assert np.allclose(oracle.gemm_fprop_ref_at(qx, sx, qw, sw, rows, cols), full[np.ix_(rows, cols)], rtol=1e-14)
    qdy = rand_codes(rng, (M, N))
    sdy = rng.uniform(0.01, 1, size=(N // 128, M)).astype(np.float32)
    qw2 = rand_codes(rng, (N, K))
    full = oracle.gemm_dgrad_ref(qdy, sdy, qw2, sw)
    cols2 = np.array([0, 200, 383])
    assert np.allclose(oracle.gemm_dgrad_ref_at(qdy, sdy, qw2, sw, rows, cols2), full[np.ix_(rows, cols2)], rtol=1e-14)
    Mt = 256
    qdyt, qxt = rand_codes(rng, (N, Mt)), rand_codes(rng, (K, Mt))
    sdyt = rng.uniform(0.01, 1, size=(Mt // 128, N)).astype(np.float32)
    sxt = rng.uniform(0.01, 1, size=(Mt // 128, K)).astype(np.float32)
    full = oracle.gemm_wgrad_ref(qdyt, sdyt, qxt, sxt)
    assert np.allclose(oracle.gemm_wgrad_ref_at(qdyt, sdyt, qxt, sxt, rows[:2], cols2), full[np.ix_(rows[:2], cols2)], rtol=1e-14)


def test_linearity_in_weight_scale():
    rng = np.random.default_rng(6)
    qx, qw = rand_codes(rng, (4, 256)), rand_codes(rng, (128, 256))
    sx = rng.uniform(0.01, 1, size=(2, 4)).astype(np.float32)
    sw = rng.uniform(0.01, 1, size=(1, 2)).astype(np.float32)
    a = oracle.gemm_fprop_ref(qx, sx, qw, sw)
    b = oracle.gemm_fprop_ref(qx, sx, qw, sw * np.float32(2))
    assert np.array_equal(b, 2 * a)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-30, 30, 10000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 2.0 ** -130]])
    got = oracle.f64_to_bf16_bits(v)
    want = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # ties to even by hand: 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7 -> 1.0 (0x3f80)
    assert got[-3] == 0x3F80 and got[-2] == 0x3F82


def test_check_gemm_tolerance():
    rng = np.random.default_rng(8)
    ref = rng.standard_normal((64, 64))
    yb = oracle.f64_to_bf16_bits(ref)
    r = oracle.check_gemm(yb, ref)
    assert r["ok"] and r["normwise"] == 0.0
    # one element off by one bf16 ulp: still within the elementwise bound
    y1 = yb.copy()
    y1[3, 4] += 1
    assert oracle.check_gemm(y1, ref)["ok"]
    # one element off by 50 ulp of a mid-size value: elementwise failure
    y2 = yb.copy()
    y2[3, 4] = oracle.f64_to_bf16_bits(np.array(ref[3, 4] + 0.05))
    assert not oracle.check_gemm(y2, ref)["ok"]
    # a uniform 0.4 % relative error fails the normwise bound
    y3 = oracle.f64_to_bf16_bits(ref * 1.004)
    assert not oracle.check_gemm(y3, ref)["ok"]
    # zero reference needs an exactly zero result
    z = np.zeros((4, 4))
    assert oracle.check_gemm(oracle.f64_to_bf16_bits(z), z)["ok"]
    assert not oracle.check_gemm(np.full((4, 4), 1, np.uint16), z)["ok"]
    assert np.array_equal(oracle.bf16_ulp(np.array([1.0, 1.5, 2.0 ** -130, 0.0])),
                          np.array([2.0 ** -7, 2.0 ** -7, 2.0 ** -133, 2.0 ** -133]))


def test_check_gemm_f32_tolerance():
    rng = np.random.default_rng(9)
    ref = rng.standard_normal((64, 64))
    y = ref.astype(np.float32)
    r = oracle.check_gemm_f32(y, ref)
    assert r["ok"] and r["normwise"] < 1e-7
    # one element just inside / just outside ulp_bf16(ref) + 1e-3 rms
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bound = float(oracle.bf16_ulp(ref[5, 6])) + 1e-3 * rms
    y1 = y.copy()
    y1[5, 6] = np.float32(ref[5, 6] + 0.98 * bound)
    assert oracle.check_gemm_f32(y1, ref)["ok"]
    y1[5, 6] = np.float32(ref[5, 6] - 1.05 * bound)
    assert not oracle.check_gemm_f32(y1, ref)["ok"]
    # a uniform 0.2 % relative error fails the normwise bound
    assert not oracle.check_gemm_f32((ref * 1.002).astype(np.float32), ref)["ok"]
    # accumulation: the bound follows the added product, not the (large) base value
    base = rng.standard_normal((64, 64)) * 1e3
    tot = base + ref
    assert oracle.check_gemm_f32(tot.astype(np.float32), tot, contrib64=ref)["ok"]
    yw = tot.astype(np.float32)
    yw[1, 2] += np.float32(0.25)  # far beyond the product's bound, far below the base's bf16 ulp
    assert not oracle.check_gemm_f32(yw, tot, contrib64=ref)["ok"]
    # zero product: the result must equal the reference exactly
    z = np.zeros((4, 4))
    assert oracle.check_gemm_f32(z.astype(np.float32), z)["ok"]
    assert not oracle.check_gemm_f32(np.full((4, 4), 1e-30, np.float32), z)["ok"]
