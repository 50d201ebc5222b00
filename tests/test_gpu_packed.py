"""GPU parity of the rollout-packed weight path: pack_weight_rollout against the
oracle's byte order, and gemm_fprop_packed against gemm_fprop (bit for bit) and
the fp64 oracle, through the C ABI.

The packed FProp reads the same codes through the same lane fragments and folds
the same block products in the same order as the row-major decode kernel, so a
row's output must equal gemm_fprop's exactly; the oracle check applies the
GEMM acceptance (normwise 1e-3, elementwise ulp_bf16 + 1e-3 rms).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Guarded, f32_dev, host, u8_dev
import quantized_rl_amd as jet
from test_gpu_gemm import check, codes, scales

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (384, 1152), (6144, 4096), (4096, 12288)])
def test_pack_matches_oracle(n, k):
    rng = np.random.default_rng(n + 7 * k)
    qw = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    g = Guarded((n, k), torch.uint8)
    jet.pack_weight_rollout(u8_dev(qw), g.t)
    torch.cuda.synchronize()
    assert g.intact()
    assert np.array_equal(host(g.t), oracle.pack_weight_rollout(qw))


def test_pack_empty():
    for n, k in [(0, 256), (128, 0)]:
        out = jet.pack_weight_rollout(torch.zeros((n, k), dtype=torch.uint8, device="cuda"))
        assert out.shape == (n, k)
    torch.cuda.synchronize()


@pytest.mark.parametrize("k", [128, 512, 4096, 8192])
@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 50, 64])
@pytest.mark.parametrize("n", [384, 6144])
def test_fprop_packed_equals_fprop(n, m, k):
    """M = 1 .. 64 (one or two token sub-tiles per wave, in one or more grid rows
    of 16 or 32 tokens; ragged 5 / 17 / 33 / 50), K = 1 .. 64 blocks (waves per
    strip group 1 .. 16, so grid rows also meet the LDS fold), N = 384 (one strip
    per wave) and 6144 (two): bitwise gemm_fprop, output guards intact, and the
    oracle's acceptance."""
    rng = np.random.default_rng(5000 + 11 * m + k + n)
    qx, qw = codes(rng, (m, k)), codes(rng, (n, k))
    sx, sw = scales(rng, (k // 128, m)), scales(rng, (n // 128, k // 128))
    qx_d, sx_d, qw_d, sw_d = u8_dev(qx), f32_dev(sx), u8_dev(qw), f32_dev(sw)
    qwp = jet.pack_weight_rollout(qw_d)
    yg = Guarded((m, n), torch.bfloat16)
    jet.gemm_fprop_packed(qx_d, sx_d, qwp, sw_d, yg.t)
    y_row = host(jet.gemm_fprop(qx_d, sx_d, qw_d, sw_d))
    torch.cuda.synchronize()
    assert yg.intact()
    y = host(yg.t)
    assert np.array_equal(y, y_row), f"packed vs row-major {m}x{n}x{k}"
    if k <= 4096:
        check(y, oracle.gemm_fprop_ref(qx, sx, qw, sw), f"packed fprop {m}x{n}x{k}")


@pytest.mark.parametrize("name,n,k", [("qkv", 6144, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)])
@pytest.mark.parametrize("m", [16, 32, 64])
def test_fprop_packed_8b_rollout_shapes(name, n, k, m):
    """The Qwen3-8B rollout projections at the decode batch sizes the benchmark
    times: bitwise gemm_fprop over the whole output, and the oracle on 8 sampled
    rows x 64 sampled columns."""
    rng = np.random.default_rng(6000 + m + n // 128)
    qx, qw = codes(rng, (m, k)), codes(rng, (n, k))
    sx, sw = scales(rng, (k // 128, m)), scales(rng, (n // 128, k // 128))
    qx_d, sx_d, qw_d, sw_d = u8_dev(qx), f32_dev(sx), u8_dev(qw), f32_dev(sw)
    y_p = host(jet.gemm_fprop_packed(qx_d, sx_d, jet.pack_weight_rollout(qw_d), sw_d))
    y_r = host(jet.gemm_fprop(qx_d, sx_d, qw_d, sw_d))
    assert np.array_equal(y_p, y_r), name
    rows = np.sort(rng.choice(m, size=min(m, 8), replace=False))
    cols = np.sort(rng.choice(n, size=64, replace=False))
    ref = oracle.gemm_fprop_ref_at(qx, sx, qw, sw, rows, cols)
    check(y_p[np.ix_(rows, cols)], ref, f"{name} m={m} sampled")


def test_fprop_packed_k_zero_and_empty():
    qx = torch.zeros((8, 0), dtype=torch.uint8, device="cuda")
    sx = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    qwp = torch.zeros((256, 0), dtype=torch.uint8, device="cuda")
    sw = torch.zeros((2, 0), dtype=torch.float32, device="cuda")
    y = torch.full((8, 256), 1.5, dtype=torch.bfloat16, device="cuda")
    jet.gemm_fprop_packed(qx, sx, qwp, sw, y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    y0 = jet.gemm_fprop_packed(torch.zeros((0, 128), dtype=torch.uint8, device="cuda"),
                               torch.zeros((1, 0), dtype=torch.float32, device="cuda"),
                               torch.zeros((256, 128), dtype=torch.uint8, device="cuda"),
                               torch.ones((2, 1), dtype=torch.float32, device="cuda"))
    assert y0.shape == (0, 256)
