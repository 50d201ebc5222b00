"""GPU parity of the RMSNorm backward (rmsnorm_backward) and of the forward's
saved factor (rmsnorm_quant_rstd) against the oracle.

rstd is a chain of fp32 operations, so it must match the oracle bit for bit,
and rmsnorm_quant_rstd's codes and scales must equal rmsnorm_quant's.  The
gradients are checked with oracle.check_rmsnorm_backward (bounds derived from
the fp32 arithmetic against the fp64 derivatives).  Inputs follow the decode
and training workloads: x ~ N(0, 1) (the training batch with its x50 outlier
channels), gamma ~ N(1, 0.05), dy ~ N(0, 1e-3) like the configs' dY.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Guarded, bf16_dev, host
import quantized_rl_amd as jet
from quantized_rl_amd import synth

pytestmark = pytest.mark.gpu

EPS = 1e-6


def gamma_bits(k, seed):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((1 + 0.05 * rng.standard_normal(k)).astype(np.float32))


@pytest.mark.parametrize("m,k", [(1, 128), (5, 640), (64, 4096), (3, 7808), (2, 12288)])
def test_rstd_forward_bit_exact(m, k):
    x = synth.random_bf16((m, k), seed=m + k)
    g = gamma_bits(k, seed=k)
    q, s, r = jet.rmsnorm_quant_rstd(bf16_dev(x), bf16_dev(g), EPS)
    q0, s0 = jet.rmsnorm_quant(bf16_dev(x), bf16_dev(g), EPS)
    assert torch.equal(q, q0) and torch.equal(s, s0)
    assert np.array_equal(host(r).view(np.uint32), oracle.rmsnorm_rstd_f32(x, EPS).view(np.uint32))


def run_backward(x, g, dy):
    xd, gd, dyd = bf16_dev(x), bf16_dev(g), bf16_dev(dy)
    _, _, r = jet.rmsnorm_quant_rstd(xd, gd, EPS)
    m, k = x.shape
    dx = Guarded((m, k), torch.bfloat16)
    dg = Guarded((k,), torch.float32)
    ws = torch.full((max(jet.rmsnorm_backward_workspace_bytes(m, k) // 4, 1),), float("nan"),
                    dtype=torch.float32, device="cuda:0")  # contents on entry are ignored
    jet.rmsnorm_backward(xd, gd, r, dyd, dx=dx.t, dgamma=dg.t, workspace=ws)
    torch.cuda.synchronize()
    assert dx.intact() and dg.intact()
    return host(dx.t), host(dg.t)


# ragged row counts (not a multiple of a workgroup's rows), K not a multiple of
# 512 (a partial last pass) or of 2048 (waves with fewer passes), the 8B and 32B
# hidden sizes, and widths past 6144 (eight and sixteen waves per row, up to the
# 24576 limit)
@pytest.mark.parametrize("m,k", [(1, 128), (31, 384), (33, 640), (64, 4096), (100, 5120), (257, 6144), (1500, 2560),
                                 (65, 6272), (40, 8192), (70, 12800), (9, 14336), (3, 24576)])
def test_rmsnorm_backward_matches_oracle(m, k):
    print(f"[rmsnorm_backward] m={m} k={k}", flush=True)
    x = synth.random_bf16((m, k), seed=7 * m + k)
    g = gamma_bits(k, seed=k + 1)
    dy = synth.random_bf16((m, k), seed=11 * m + k, std=1e-3)
    dx, dg = run_backward(x, g, dy)
    r = oracle.check_rmsnorm_backward(dx, dg, x, g, dy, EPS)
    assert r["ok"], r


def test_rmsnorm_backward_training_batch():
    """The 8B training batch (8192 x 4096 with outlier channels): every output
    against the oracle, and a second call gives the same bits."""
    d = synth.linear_8b_up()
    x = d["x"]
    m, k = x.shape
    print(f"[rmsnorm_backward] m={m} k={k}", flush=True)
    g = gamma_bits(k, seed=5)
    dy = synth.random_bf16((m, k), seed=6, std=1e-3)
    dx, dg = run_backward(x, g, dy)
    r = oracle.check_rmsnorm_backward(dx, dg, x, g, dy, EPS)
    assert r["ok"], r
    dx2, dg2 = run_backward(x, g, dy)
    assert np.array_equal(dx, dx2) and np.array_equal(dg.view(np.uint32), dg2.view(np.uint32))


def test_rmsnorm_backward_zero_rows_and_zero_gradient():
    """An all-zero x row (rstd = eps^-1/2, dx = rstd * gamma * dy) and an all-zero dy
    (dx = 0, dgamma = 0); M = 0 writes dgamma = 0."""
    m, k = 40, 512
    x = synth.random_bf16((m, k), seed=1)
    x[3] = 0
    g = gamma_bits(k, seed=2)
    dy = synth.random_bf16((m, k), seed=3, std=1e-3)
    dx, dg = run_backward(x, g, dy)
    assert oracle.check_rmsnorm_backward(dx, dg, x, g, dy, EPS)["ok"]
    dx0, dg0 = run_backward(x, g, np.zeros_like(dy))
    assert not np.any(dx0 & 0x7FFF) and not np.any(dg0)
    e8 = torch.empty((0, k), dtype=torch.bfloat16, device="cuda:0")
    dgz = torch.full((k,), 7.0, dtype=torch.float32, device="cuda:0")
    jet.rmsnorm_backward(e8, bf16_dev(g), torch.empty((0,), dtype=torch.float32, device="cuda:0"), e8,
                         dgamma=dgz)
    assert bool((dgz == 0).all())


def test_rmsnorm_fp8_linear_block_chains_the_kernels():
    """RMSNormFP8Linear: the forward equals rmsnorm_quant + gemm_fprop (FP8 codes
    bit-exact against the oracle), and the backward's x / gamma gradients are
    rmsnorm_backward applied to the GEMM's DGrad output -- checked against the
    oracle with that bf16 DGrad output as the upstream gradient."""
    from quantized_rl_amd import linear
    m, k, n = 256, 512, 384
    torch.manual_seed(3)
    blk = linear.RMSNormFP8Linear(k, n, device=torch.device("cuda:0"))
    with torch.no_grad():
        blk.gamma.copy_(bf16_dev(gamma_bits(k, seed=9)))
    x_h = synth.random_bf16((m, k), seed=21)
    dy_h = synth.random_bf16((m, n), seed=22, std=1e-3)
    x = bf16_dev(x_h).requires_grad_(True)
    y = blk(x)
    y.backward(bf16_dev(dy_h))
    torch.cuda.synchronize()
    g_h = host(blk.gamma.detach())
    w = blk.weight.detach()
    # forward: the norm's codes and the GEMM
    qx, sx = jet.rmsnorm_quant(bf16_dev(x_h), blk.gamma.detach(), blk.eps)
    qxo, sxo = oracle.rmsnorm_quant(x_h, g_h, blk.eps)
    assert np.array_equal(host(qx), qxo) and np.array_equal(host(sx), sxo)
    qw, sw = jet.quantize_weight_128x128(w)
    assert torch.equal(y.detach(), jet.gemm_fprop(qx, sx, qw, sw))
    # backward: DGrad output (bf16) -> RMSNorm gradients
    qdy, sdy = jet.quantize_act_1x128(bf16_dev(dy_h))
    dxn = jet.gemm_dgrad(qdy, sdy, qw, sw)
    rstd = jet.rmsnorm_quant_rstd(bf16_dev(x_h), blk.gamma.detach(), blk.eps)[2]
    dx_ref, dg32 = jet.rmsnorm_backward(bf16_dev(x_h), blk.gamma.detach(), rstd, dxn)
    assert torch.equal(x.grad, dx_ref)
    # gamma's bf16 gradient is the rounding of the fp32 one
    assert torch.equal(blk.gamma.grad, dg32.to(torch.bfloat16))
    r = oracle.check_rmsnorm_backward(host(x.grad), host(dg32), x_h, g_h, host(dxn), blk.eps)
    assert r["ok"], r
    assert blk.weight.grad is not None and bool(torch.isfinite(blk.weight.grad.float()).all())
