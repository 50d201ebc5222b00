"""Seeded random shapes across every GEMM launch rule, against the fp64 oracle.

The hand-picked shapes of test_gpu_gemm.py and test_gpu_packed.py sit on the
launch rules' boundaries; here a fixed-seed draw of (M, N, K) spreads over all
of them at once (rollout batches of 1 .. 256 tokens, the 128 x 128 and
256 x 256 tile kernels, weights wide enough for the six-strip weight-sharing
shape, contractions from one to 96 K-blocks).  Per FProp shape: the output
against the oracle, the packed-weight FProp bitwise equal to it (up to 256
rows), and a leading slice of its rows bitwise equal to the same rows run as a
batch of their own (another kernel for most shapes: the fold is the same).
DGrad and WGrad shapes: the output against the oracle.  Operands are the
quantised-Gaussian codes and scales of test_gpu_gemm; acceptance is the GEMM
contract (normwise 1e-3, elementwise ulp_bf16 + 1e-3 rms)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Guarded, f32_dev, host, u8_dev
import quantized_rl_amd as jet
from test_gpu_gemm import check, codes, scales

pytestmark = pytest.mark.gpu

_MAX_MNK = 1.2e10  # the oracle finishes a case in about a second


def _draw(seed, count, kind):
    """count shapes (M, N, K) in the argument order of the kind's test; about a
    quarter of them give the 256 x 256 kernel at least 256 output tiles."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        band = rng.integers(0, 4)
        if kind == "wgrad":
            m = 128 * int(rng.integers(1, 24))
        elif band == 0:
            m = int(rng.integers(1, 33))
        elif band == 1:
            m = int(rng.integers(33, 257))
        elif band == 2:
            m = int(rng.integers(257, 1200))
        else:
            m = int(rng.integers(1200, 4200))
        wide = rng.random() < 0.15
        n = 128 * (192 * int(rng.integers(1, 3)) if wide else int(rng.integers(1, 49)))
        k = 128 * (int(rng.integers(65, 97)) if rng.random() < 0.15 else int(rng.integers(1, 41)))
        if band == 3:  # the 256 x 256 kernel: a wide output, a short contraction
            wide_out, short = 256 * int(rng.integers(8, 49)), 128 * int(rng.integers(1, 5))
            if kind == "fprop":
                n, k = wide_out, short
            elif kind == "dgrad":
                n, k = short, wide_out
            else:
                m, n, k = 128 * int(rng.integers(1, 5)), 256 * int(rng.integers(16, 49)), wide_out
        if m * n * k <= _MAX_MNK:
            out.append((m, n, k))
    return out


FPROP = _draw(20261203, 28, "fprop")
DGRAD = _draw(20261204, 16, "dgrad")
WGRAD = _draw(20261205, 16, "wgrad")


@pytest.mark.parametrize("m,n,k", FPROP)
def test_fprop_shape_sweep(m, n, k):
    print(f"[shape sweep] fprop {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng(m * 131 + n * 7 + k)
    qx, qw = codes(rng, (m, k)), codes(rng, (n, k))
    sx, sw = scales(rng, (k // 128, m)), scales(rng, (n // 128, k // 128))
    dqx, dsx, dqw, dsw = u8_dev(qx), f32_dev(sx), u8_dev(qw), f32_dev(sw)
    yg = Guarded((m, n), torch.bfloat16)
    jet.gemm_fprop(dqx, dsx, dqw, dsw, yg.t)
    torch.cuda.synchronize()
    assert yg.intact()
    y = host(yg.t)
    check(y, oracle.gemm_fprop_ref(qx, sx, qw, sw), f"fprop {m}x{n}x{k}")
    if m <= 256:
        yp = host(jet.gemm_fprop_packed(dqx, dsx, jet.pack_weight_rollout(dqw), dsw))
        assert np.array_equal(yp, y), f"packed fprop {m}x{n}x{k}"
    r = min(m, 40)
    ys = host(jet.gemm_fprop(dqx[:r].contiguous(), dsx[:, :r].contiguous(), dqw, dsw))
    assert np.array_equal(ys, y[:r]), f"first {r} rows of fprop {m}x{n}x{k} as a batch of their own"


@pytest.mark.parametrize("m,n,k", DGRAD)
def test_dgrad_shape_sweep(m, n, k):
    print(f"[shape sweep] dgrad {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng(m * 131 + n * 5 + k)
    qdy, qw = codes(rng, (m, n)), codes(rng, (n, k))
    sdy, sw = scales(rng, (n // 128, m)), scales(rng, (n // 128, k // 128))
    dg = Guarded((m, k), torch.bfloat16)
    jet.gemm_dgrad(u8_dev(qdy), f32_dev(sdy), u8_dev(qw), f32_dev(sw), dg.t)
    torch.cuda.synchronize()
    assert dg.intact()
    check(host(dg.t), oracle.gemm_dgrad_ref(qdy, sdy, qw, sw), f"dgrad {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", WGRAD)
def test_wgrad_shape_sweep(m, n, k):
    print(f"[shape sweep] wgrad {m}x{n}x{k}", flush=True)
    rng = np.random.default_rng(m * 131 + n * 3 + k)
    qdyt, qxt = codes(rng, (n, m)), codes(rng, (k, m))
    sdyt, sxt = scales(rng, (m // 128, n)), scales(rng, (m // 128, k))
    dg = Guarded((n, k), torch.bfloat16)
    jet.gemm_wgrad(u8_dev(qdyt), f32_dev(sdyt), u8_dev(qxt), f32_dev(sxt), dg.t)
    torch.cuda.synchronize()
    assert dg.intact()
    check(host(dg.t), oracle.gemm_wgrad_ref(qdyt, sdyt, qxt, sxt), f"wgrad {m}x{n}x{k}")
