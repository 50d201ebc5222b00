"""Backward of the RMSNorm in front of the FP8 linear (oracle; test infra only).

The pages name a fused RMSNorm in the forward (page paper.rainbus.top/paper/
2601.14243, section "方法步骤详情", step 5) and train through it, but give no
formula for either direction.  The forward read here is the standard RMSNorm,
y = x * gamma * rho with rho = (mean_k x_k^2 + eps)^(-1/2) per row.  Its
gradients, for an upstream gradient dy, follow from calculus on that real
function:

    dgamma_k = sum_m dy_mk * x_mk * rho_m
    dx_mk    = rho_m * (gamma_k * dy_mk - x_mk * rho_m^2 * c_m),
    c_m      = (1 / K) * sum_j gamma_j * dy_mj * x_mj.

The reference evaluates these in fp64 from the exact bf16 inputs, with eps
rounded to fp32 as the forward uses it.  Parity of the GPU result is checked
to a tolerance derived from its fp32 arithmetic (see check_rmsnorm_backward).
"""

import numpy as np

from .gemm import bf16_bits_to_f64, bf16_ulp


def rmsnorm_backward_ref(x_bf16, gamma_bf16, dy_bf16, eps):
    """(dx f64 [M, K], dgamma f64 [K], rho f64 [M]) for bf16 x [M, K], gamma [K], dy [M, K]."""
    x = bf16_bits_to_f64(x_bf16)
    g = bf16_bits_to_f64(gamma_bf16)
    dy = bf16_bits_to_f64(dy_bf16)
    if x.ndim != 2 or dy.shape != x.shape or g.shape != (x.shape[1],) or x.shape[1] == 0:
        raise ValueError("expected x, dy [M, K] and gamma [K], K > 0")
    if not (np.all(np.isfinite(x)) and np.all(np.isfinite(g)) and np.all(np.isfinite(dy))):
        raise ValueError("inputs must be finite")
    k = x.shape[1]
    e = float(np.float32(eps))
    rho = 1.0 / np.sqrt(np.mean(x * x, axis=1) + e)
    c = np.sum(g[None, :] * dy * x, axis=1) / k
    dx = rho[:, None] * (g[None, :] * dy - x * (rho * rho * c)[:, None])
    dgamma = np.sum(dy * x * rho[:, None], axis=0)
    return dx, dgamma, rho


def check_rmsnorm_backward(dx_bf16, dgamma_f32, x_bf16, gamma_bf16, dy_bf16, eps):
    """Acceptance of a GPU RMSNorm backward (dx bf16 bits [M, K], dgamma fp32 [K]).

    The GPU works in fp32 from the forward's fp32 rho (relative error <= 2^-23)
    with a handful of roundings per element and fp32 sums: over a row for c
    (at most K terms) and over the rows for dgamma (at most a few hundred terms
    per partial plus the partials).  Bounds, with u = 2^-24 and generous
    margins over those operation counts:
      |dx - dx64|         <= ulp_bf16(dx64) + 2^-14 * rho * (|gamma dy| + |x| rho^2 c_abs),
                             c_abs = (1/K) sum_j |gamma_j dy_j x_j|;
      |dgamma - dgamma64| <= 2^-12 * sum_m |dy_mk x_mk rho_m|.
    (2^-14 is 1024 u, 2^-12 is 4096 u.)  Returns a dict with the worst excess of
    each bound and 'ok'.
    """
    x = bf16_bits_to_f64(x_bf16)
    g = bf16_bits_to_f64(gamma_bf16)
    dy = bf16_bits_to_f64(dy_bf16)
    dx64, dg64, rho = rmsnorm_backward_ref(x_bf16, gamma_bf16, dy_bf16, eps)
    k = x.shape[1]
    c_abs = np.sum(np.abs(g[None, :] * dy * x), axis=1) / k
    bound_dx = bf16_ulp(dx64) + 2.0 ** -14 * rho[:, None] * (
        np.abs(g[None, :] * dy) + np.abs(x) * (rho * rho * c_abs)[:, None])
    dx = bf16_bits_to_f64(dx_bf16)
    ex_dx = float(np.max(np.abs(dx - dx64) - bound_dx)) if dx.size else -1.0
    bound_dg = 2.0 ** -12 * np.sum(np.abs(dy * x * rho[:, None]), axis=0)
    dg = np.asarray(dgamma_f32, dtype=np.float32).astype(np.float64)
    ex_dg = float(np.max(np.abs(dg - dg64) - bound_dg)) if dg.size else -1.0
    return {"ok": bool(ex_dx <= 0.0 and ex_dg <= 0.0), "dx_excess": ex_dx, "dgamma_excess": ex_dg}
