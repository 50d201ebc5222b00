"""GPU parity of the rollout-packed weight path: pack_weight_rollout against the
oracle's byte order, and gemm_fprop_packed against gemm_fprop (bit for bit) and
the fp64 oracle, through the C ABI.

The packed FProp reads the same codes through the same lane fragments and folds
the same block products in the same order as gemm_fprop's kernels, so a row's
output must equal gemm_fprop's exactly, in the same batch or inside a training
batch of more than 256 rows; the oracle check applies the GEMM acceptance
(normwise 1e-3, elementwise ulp_bf16 + 1e-3 rms).
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


BATCH = 300  # a training-size batch: gemm_fprop's 128 x 128 kernel


def packed_case(rng, m, n, k):
    """Codes and scales of a BATCH-row X whose first m rows are the case's, the
    weight, and the packed and row-major outputs: packed over the m rows (guards
    checked), row-major over the m rows and over the whole batch."""
    qx, qw = codes(rng, (BATCH, k)), codes(rng, (n, k))
    sx, sw = scales(rng, (k // 128, BATCH)), scales(rng, (n // 128, k // 128))
    sxm = np.ascontiguousarray(sx[:, :m])
    qx_d, sx_d, qw_d, sw_d = u8_dev(qx[:m]), f32_dev(sxm), u8_dev(qw), f32_dev(sw)
    yg = Guarded((m, n), torch.bfloat16)
    jet.gemm_fprop_packed(qx_d, sx_d, jet.pack_weight_rollout(qw_d), sw_d, yg.t)
    y_row = host(jet.gemm_fprop(qx_d, sx_d, qw_d, sw_d))
    y_big = host(jet.gemm_fprop(u8_dev(qx), f32_dev(sx), qw_d, sw_d))[:m]
    torch.cuda.synchronize()
    assert yg.intact()
    return qx[:m], sxm, qw, sw, host(yg.t), y_row, y_big


@pytest.mark.parametrize("k", [128, 512, 4096, 8192])
@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 50, 64, 65, 100, 128, 200, 256])
@pytest.mark.parametrize("n", [384, 6144])
def test_fprop_packed_equals_fprop(n, m, k):
    """M = 1 .. 64 through the decode kernel (one or two token sub-tiles per wave,
    in one or more grid rows of 16 or 32 tokens; ragged 5 / 17 / 33 / 50) or, from
    33 rows, the weight-sharing kernel (token groups of 64 or 128 rows, ragged 100
    and 200, with 1 .. 6 strips per workgroup), K = 1 .. 64 blocks, N = 384 and
    6144: bitwise gemm_fprop on the same rows and inside a 300-row batch, output
    guards intact, and the oracle's acceptance."""
    rng = np.random.default_rng(5000 + 11 * m + k + n)
    qx, sx, qw, sw, y, y_row, y_big = packed_case(rng, m, n, k)
    assert np.array_equal(y, y_row), f"packed vs row-major {m}x{n}x{k}"
    assert np.array_equal(y, y_big), f"packed vs training batch {m}x{n}x{k}"
    if k <= 4096 and m * n * k <= 256 * 6144 * 512:
        check(y, oracle.gemm_fprop_ref(qx, sx, qw, sw), f"packed fprop {m}x{n}x{k}")
    elif k <= 4096:
        rows = np.sort(rng.choice(m, size=min(m, 12), replace=False))
        cols = np.sort(rng.choice(n, size=96, replace=False))
        check(y[np.ix_(rows, cols)], oracle.gemm_fprop_ref_at(qx, sx, qw, sw, rows, cols),
              f"packed fprop {m}x{n}x{k} sampled")


@pytest.mark.parametrize("k", [128, 1024])
@pytest.mark.parametrize("m", [33, 64, 100, 128, 200, 256])
def test_fprop_packed_six_strip_groups(m, k):
    """N = 24576 (1536 strips of 16 columns, the 8B gate+up width): the
    weight-sharing kernel's 6-strip workgroups, most of which span two
    128-column weight blocks, with all rows in one token group (4 waves of 16 or
    32 tokens, 8 waves of 32 over 128 rows).  Bitwise gemm_fprop and the
    training batch over the whole output; the oracle on sampled rows and on
    every column of three workgroups that cross a weight-block boundary."""
    n = 24576
    rng = np.random.default_rng(5500 + m + k)
    qx, sx, qw, sw, y, y_row, y_big = packed_case(rng, m, n, k)
    assert np.array_equal(y, y_row) and np.array_equal(y, y_big), f"{m}x{n}x{k}"
    rows = np.sort(rng.choice(m, size=min(m, 10), replace=False))
    cols = np.concatenate([np.arange(96 * g, 96 * g + 96) for g in (1, 2, 3)])  # columns 96 .. 383
    check(y[np.ix_(rows, cols)], oracle.gemm_fprop_ref_at(qx, sx, qw, sw, rows, cols), f"{m}x{n}x{k} sampled")


def test_fprop_packed_long_contraction_fallback():
    """More than 512 K-blocks (K = 66048): the weight-sharing kernel's copy of the
    weight-block scales would not fit, so 100 rows run the decode kernel; still
    bitwise gemm_fprop (whose 100-row batch then runs the 128 x 128 kernel) and
    within the oracle's acceptance."""
    m, n, k = 100, 128, 66048
    rng = np.random.default_rng(5600)
    qx, sx, qw, sw, y, y_row, y_big = packed_case(rng, m, n, k)
    assert np.array_equal(y, y_row) and np.array_equal(y, y_big)
    check(y, oracle.gemm_fprop_ref(qx, sx, qw, sw), f"packed fprop {m}x{n}x{k}")


@pytest.mark.parametrize("name,n,k", [("qkv", 6144, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)])
@pytest.mark.parametrize("m", [16, 32, 64, 128, 256])
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
