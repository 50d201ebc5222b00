"""GPU parity of gemm_wgrad_f32 (the weight gradient kept in fp32, written or
added to an existing fp32 gradient) against the fp64 oracle.

Acceptance (oracle.check_gemm_f32): the bf16 result's bound against the unrounded
reference, normwise ||Y - Yref64|| / ||G64|| <= 1e-3 and elementwise
|Y - Yref64| <= ulp_bf16(G64) + 1e-3 rms(G64) + 2^-23 |Yref64|, G64 being the product.
Beyond that the fp32 result is tied to the bf16 entry point bit for bit: gemm_wgrad's
output is the nearest-even bf16 rounding of it, and accumulate=1 adds it to the
old value in one fp32 addition.  Exact-integer cases match the oracle exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Guarded, bf16_dev, f32_dev, grouped_cols, host, requant_cols_deq, u8_dev
import quantized_rl_amd as jet
from quantized_rl_amd import synth
from test_gpu_gemm import codes, scales

pytestmark = pytest.mark.gpu

# (M tokens, N rows of dW, K columns): the medium-tile kernel, and (last two)
# the 256 x 256 kernel with a ragged last row tile (6528 = 25.5 x 256; a last round of more
# than half the CUs, so every tile stays on that kernel)
SHAPES = [(128, 128, 128), (256, 384, 512), (1024, 1280, 512), (256, 6528, 4096), (384, 6528, 4096)]


def operands(m, n, k, seed, small=False):
    rng = np.random.default_rng(seed)
    qdyt, qxt = codes(rng, (n, m), small=small), codes(rng, (k, m), small=small)
    sdyt, sxt = scales(rng, (m // 128, n), pow2=small), scales(rng, (m // 128, k), pow2=small)
    return qdyt, sdyt, qxt, sxt


def dev(qdyt, sdyt, qxt, sxt):
    return u8_dev(qdyt), f32_dev(sdyt), u8_dev(qxt), f32_dev(sxt)


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_wgrad_f32_matches_oracle_and_bf16_entry_point(m, n, k):
    print(f"[wgrad_f32] m={m} n={n} k={k}", flush=True)
    ops = operands(m, n, k, seed=m + 7 * n + k)
    d = dev(*ops)
    g = Guarded((n, k), torch.float32)
    jet.gemm_wgrad_f32(*d, dw=g.t)
    dw16 = jet.gemm_wgrad(*d)
    torch.cuda.synchronize()
    assert g.intact()
    y = host(g.t)
    # the bf16 entry point returns exactly the nearest-even rounding of this accumulator
    assert np.array_equal(host(dw16), oracle.f64_to_bf16_bits(y.astype(np.float64)))
    r = oracle.check_gemm_f32(y, oracle.gemm_wgrad_ref(*ops))
    assert r["ok"], r


@pytest.mark.parametrize("m,n,k", [(256, 384, 512), (256, 6528, 4096)])
def test_wgrad_f32_accumulates(m, n, k):
    print(f"[wgrad_f32 accumulate] m={m} n={n} k={k}", flush=True)
    ops = operands(m, n, k, seed=3 * m + n + k)
    d = dev(*ops)
    g_only = host(jet.gemm_wgrad_f32(*d))
    rng = np.random.default_rng(5)
    base = (rng.standard_normal((n, k)) * float(np.abs(g_only).max())).astype(np.float32)
    acc = Guarded((n, k), torch.float32)
    acc.t.copy_(torch.from_numpy(base))
    jet.gemm_wgrad_f32(*d, dw=acc.t, accumulate=True)
    torch.cuda.synchronize()
    assert acc.intact()
    y = host(acc.t)
    # one fp32 addition of the same accumulator (numpy float32 add is IEEE nearest-even)
    assert np.array_equal(y, base + g_only)
    g64 = oracle.gemm_wgrad_ref(*ops)
    r = oracle.check_gemm_f32(y, base.astype(np.float64) + g64, contrib64=g64)
    assert r["ok"], r


@pytest.mark.parametrize("m,n,k", [(256, 256, 384), (384, 6528, 4096)])
def test_wgrad_f32_exact_integer(m, n, k):
    """Codes in {0, +-0.5, +-1, +-2} and power-of-two scales: every partial and
    sum is exact in fp32, so the result equals the fp64 reference exactly, and
    twice accumulated equals twice the product."""
    ops = operands(m, n, k, seed=11 + m + k, small=True)
    d = dev(*ops)
    ref = oracle.gemm_wgrad_ref(*ops)
    y = jet.gemm_wgrad_f32(*d)
    assert np.array_equal(host(y).astype(np.float64), ref)
    jet.gemm_wgrad_f32(*d, dw=y, accumulate=True)
    assert np.array_equal(host(y).astype(np.float64), 2.0 * ref)


def test_wgrad_f32_no_tokens():
    """M == 0: accumulate=0 writes zeros, accumulate=1 leaves dw as it was."""
    n, k = 256, 384
    e8 = torch.empty((n, 0), dtype=torch.uint8, device="cuda:0")
    e32 = torch.empty((0, n), dtype=torch.float32, device="cuda:0")
    x8 = torch.empty((k, 0), dtype=torch.uint8, device="cuda:0")
    x32 = torch.empty((0, k), dtype=torch.float32, device="cuda:0")
    dw = torch.full((n, k), 3.5, dtype=torch.float32, device="cuda:0")
    jet.gemm_wgrad_f32(e8, e32, x8, x32, dw=dw, accumulate=True)
    assert bool((dw == 3.5).all())
    jet.gemm_wgrad_f32(e8, e32, x8, x32, dw=dw)
    assert bool((dw == 0).all())


def test_wgrad_f32_8b_up_full_size():
    """The 8B up-projection weight gradient (N=12288, K=4096, over M=8192 tokens)
    in the launch configuration the bf16 WGrad uses: the bf16 result is the
    rounding of the fp32 one everywhere, and 48 x 48 sampled entries match the
    oracle (its operands requantised from the same bf16 inputs)."""
    d = synth.linear_8b_up()
    M, K = d["x"].shape
    N = d["w"].shape[0]
    print(f"[wgrad_f32 8b] M={M} N={N} K={K}", flush=True)
    qx, sx = jet.quantize_act_1x128(bf16_dev(d["x"]))
    qdy, sdy = jet.quantize_act_1x128(bf16_dev(d["dy"]))
    qxt, sxt = jet.requant_transpose_128x1(qx, sx)
    qdyt, sdyt = jet.requant_transpose_128x1(qdy, sdy)
    y = host(jet.gemm_wgrad_f32(qdyt, sdyt, qxt, sxt))
    dw16 = host(jet.gemm_wgrad(qdyt, sdyt, qxt, sxt))
    assert np.array_equal(dw16, oracle.f64_to_bf16_bits(y.astype(np.float64)))
    rng = np.random.default_rng(3)
    cols_n, cols_k = grouped_cols(rng, N, 48), grouped_cols(rng, K, 48)
    ref = requant_cols_deq(d["dy"], cols_n) @ requant_cols_deq(d["x"], cols_k).T
    r = oracle.check_gemm_f32(y[np.ix_(cols_n, cols_k)], ref, rms=float(np.sqrt(np.mean(ref ** 2))))
    assert r["ok"], r
