"""Pins of the RMSNorm backward oracle (oracle.norm) and of the forward's rstd.

The pages give no formula for either direction, so the pins are mathematical:
central finite differences of the forward (a computation that never uses the
gradient formulas), torch's autograd of its rms_norm in float64 (a library
routine), a closed form for sum_k x_k dx_k, and homogeneity in x.
"""

import numpy as np
import pytest
import torch

import oracle
from quantized_rl_amd import synth


def bf16(a):
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def f64(u):
    return oracle.gemm.bf16_bits_to_f64(u)


def inputs(m, k, seed, eps_scale=1.0):
    rng = np.random.default_rng(seed)
    x = bf16(rng.standard_normal((m, k)) * eps_scale)
    g = bf16(1.0 + 0.05 * rng.standard_normal(k))
    dy = bf16(rng.standard_normal((m, k)) * 1e-2)
    return x, g, dy


def forward64(x, g, eps):
    """The real-valued forward in fp64: y = x * g / sqrt(mean(x^2) + eps)."""
    return x * g[None, :] / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)


def test_matches_central_finite_differences():
    m, k, eps = 3, 256, 1e-6
    xb, gb, dyb = inputs(m, k, seed=1)
    x, g, dy = f64(xb), f64(gb), f64(dyb)
    e = float(np.float32(eps))
    dx, dg, _ = oracle.rmsnorm_backward_ref(xb, gb, dyb, eps)
    loss = lambda xx, gg: float(np.sum(dy * forward64(xx, gg, e)))
    rng = np.random.default_rng(2)
    for _ in range(40):
        i, j = int(rng.integers(m)), int(rng.integers(k))
        h = 1e-6 * max(1.0, abs(x[i, j]))
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        fd = (loss(xp, g) - loss(xm, g)) / (2 * h)
        assert abs(fd - dx[i, j]) <= 1e-6 * np.max(np.abs(dx)) + 1e-9
    for j in rng.choice(k, 20, replace=False):
        h = 1e-6
        gp, gm = g.copy(), g.copy()
        gp[j] += h
        gm[j] -= h
        fd = (loss(x, gp) - loss(x, gm)) / (2 * h)
        assert abs(fd - dg[j]) <= 1e-6 * np.max(np.abs(dg)) + 1e-9


def test_matches_torch_autograd_float64():
    m, k, eps = 16, 512, 1e-6
    xb, gb, dyb = inputs(m, k, seed=3)
    dx, dg, _ = oracle.rmsnorm_backward_ref(xb, gb, dyb, eps)
    x = torch.from_numpy(f64(xb)).requires_grad_(True)
    g = torch.from_numpy(f64(gb)).requires_grad_(True)
    y = torch.nn.functional.rms_norm(x, (k,), weight=g, eps=float(np.float32(eps)))
    y.backward(torch.from_numpy(f64(dyb)))
    assert np.allclose(x.grad.numpy(), dx, rtol=1e-10, atol=1e-14 * np.abs(dx).max())
    assert np.allclose(g.grad.numpy(), dg, rtol=1e-10, atol=1e-14 * np.abs(dg).max())


def test_closed_form_of_x_dot_dx():
    """sum_k x_k dx_k = rho * S * eps / (ms + eps), S = sum_k gamma_k dy_k x_k: the
    gradient is orthogonal to x up to the eps term (y does not change along x
    when eps = 0)."""
    m, k = 8, 384
    for eps in (1e-6, 0.5, 0.0):
        xb, gb, dyb = inputs(m, k, seed=4)
        x, g, dy = f64(xb), f64(gb), f64(dyb)
        dx, _, rho = oracle.rmsnorm_backward_ref(xb, gb, dyb, eps)
        e = float(np.float32(eps))
        ms = np.mean(x * x, axis=1)
        s = np.sum(g[None, :] * dy * x, axis=1)
        lhs = np.sum(x * dx, axis=1)
        rhs = rho * s * e / (ms + e)
        assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-12 * np.abs(dx).sum())


def test_homogeneity_in_x():
    """With eps = 0, y(c x) = y(x), so dx(c x) = dx(x) / c and dgamma is unchanged;
    c = 4 keeps the bf16 inputs exact."""
    xb, gb, dyb = inputs(4, 256, seed=5)
    x4 = bf16(f64(xb) * 4.0)
    dx1, dg1, _ = oracle.rmsnorm_backward_ref(xb, gb, dyb, 0.0)
    dx4, dg4, _ = oracle.rmsnorm_backward_ref(x4, gb, dyb, 0.0)
    assert np.allclose(dx4 * 4.0, dx1, rtol=1e-12, atol=0)
    assert np.allclose(dg4, dg1, rtol=1e-12, atol=0)


def test_rstd_is_the_forward_factor():
    """rmsnorm_rstd_f32 is the factor rmsnorm_f32 applies: with gamma = 1 the
    forward output is fl32(x * rstd) bit for bit, and rstd is within 2^-21 of
    the exact fp64 value."""
    xb, _, _ = inputs(6, 640, seed=6)
    ones = bf16(np.ones(640))
    r = oracle.rmsnorm_rstd_f32(xb, 1e-6)
    y = oracle.rmsnorm_f32(xb, ones, 1e-6)
    x32 = oracle.bf16_bits_to_f32(xb)
    assert np.array_equal(y, (x32 * r[:, None]).astype(np.float32))
    exact = 1.0 / np.sqrt(np.mean(f64(xb) ** 2, axis=1) + float(np.float32(1e-6)))
    assert np.all(np.abs(r - exact) <= 2.0 ** -21 * exact)


def test_check_rmsnorm_backward_rejects_planted_errors():
    m, k, eps = 8, 256, 1e-6
    xb, gb, dyb = inputs(m, k, seed=7)
    dx, dg, _ = oracle.rmsnorm_backward_ref(xb, gb, dyb, eps)
    dxb = oracle.f64_to_bf16_bits(dx)
    dg32 = dg.astype(np.float32)
    assert oracle.check_rmsnorm_backward(dxb, dg32, xb, gb, dyb, eps)["ok"]
    # dropping the mean term (a plausible mistake) fails
    x, g, dy = f64(xb), f64(gb), f64(dyb)
    rho = 1.0 / np.sqrt(np.mean(x * x, axis=1) + float(np.float32(eps)))
    wrong = rho[:, None] * g[None, :] * dy
    assert not oracle.check_rmsnorm_backward(oracle.f64_to_bf16_bits(wrong), dg32, xb, gb, dyb, eps)["ok"]
    # one dx element off by 4 bf16 ulps fails; dgamma off by 1e-3 relative fails
    bad = dxb.copy()
    bad[2, 3] += 4
    assert not oracle.check_rmsnorm_backward(bad, dg32, xb, gb, dyb, eps)["ok"]
    assert not oracle.check_rmsnorm_backward(dxb, (dg * 1.001).astype(np.float32), xb, gb, dyb, eps)["ok"]
    with pytest.raises(ValueError):
        oracle.rmsnorm_backward_ref(xb, gb[:-1], dyb, eps)
