"""GPU parity of the quantisation kernels against the CPU oracle: bit-exact.

quantize_act_1x128, quantize_weight_128x128, rmsnorm_quant and
requant_transpose_128x1 are called through the C ABI (via the ctypes binding)
on seeded synthetic inputs with the shapes of the workloads, and every FP8 code
and fp32 scale is compared bit for bit with the oracle (at full size where the
oracle is quick, on sampled rows / blocks / token blocks otherwise).
"""

import numpy as np
import pytest
import torch

import golden_io
import oracle
from gpu_common import Guarded, bf16_dev, f32_dev, host, u8_dev
import quantized_rl_amd as jet
from quantized_rl_amd import synth

pytestmark = pytest.mark.gpu


def assert_same(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"


def quant_act_gpu(xb):
    q, s = jet.quantize_act_1x128(bf16_dev(xb))
    return host(q), host(s)


def special_rows(m, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (m, k))).astype(np.float32)
    if m > 3:
        x[0] = 0.0
        x[1] = -0.0
        x[2, :128] = np.float32(3.0e38)
        x[2, 5] = np.float32(-3.3e38)
        x[3] = x[3] * np.float32(2.0 ** -126)  # subnormal values and scales
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("m,k", [(1, 128), (3, 384), (63, 256), (65, 128), (200, 640), (256, 512)])
def test_quant_act_shapes_and_specials(m, k):
    xb = special_rows(m, k, seed=m * 1000 + k)
    q, s = quant_act_gpu(xb)
    qo, so = oracle.quant_act_1x128(xb)
    assert_same(q, qo, "q")
    assert_same(s, so, "s")


def test_quant_act_golden_groups():
    cases = golden_io.quant_cases()
    x = np.zeros((len(cases), 256), np.float32)
    for i, c in enumerate(cases):
        x[i, 128:] = np.array(c["x"], np.float32)
    q, s = quant_act_gpu(synth.f32_to_bf16_bits(x))
    for i, c in enumerate(cases):
        assert s[1, i] == np.float32(c["S"]), c["name"]
        assert np.array_equal(q[i, 128:], np.array(c["q"], np.uint8)), c["name"]


def test_quant_act_linear_small():
    d = synth.linear_small()
    q, s = quant_act_gpu(d["x"])
    qo, so = oracle.quant_act_1x128(d["x"])
    assert_same(q, qo, "q")
    assert_same(s, so, "s")


def test_quant_act_linear_8b_up_full_x_and_sampled_dy():
    d = synth.linear_8b_up()
    q, s = quant_act_gpu(d["x"])
    qo, so = oracle.quant_act_1x128(d["x"])
    assert_same(q, qo, "qx")
    assert_same(s, so, "sx")
    q, s = quant_act_gpu(d["dy"])
    rows = np.random.default_rng(0).choice(d["dy"].shape[0], 512, replace=False)
    qo, so = oracle.quant_act_1x128(d["dy"][rows])
    assert_same(q[rows], qo, "qdy rows")
    assert_same(s[:, rows], so, "sdy rows")


def test_quant_act_empty_and_guards():
    xb = special_rows(5, 256, 3)
    qg, sg = Guarded((5, 256), torch.uint8), Guarded((2, 5), torch.float32)
    jet.quantize_act_1x128(bf16_dev(xb), qg.t, sg.t)
    torch.cuda.synchronize()
    assert qg.intact() and sg.intact()
    qo, so = oracle.quant_act_1x128(xb)
    assert_same(host(qg.t), qo, "q")
    q, s = jet.quantize_act_1x128(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda:0"))
    assert q.shape == (0, 256) and s.shape == (2, 0)


def test_quant_act_deterministic():
    xb = synth.random_bf16((300, 1024), seed=5)
    a = quant_act_gpu(xb)
    b = quant_act_gpu(xb)
    assert_same(a[0], b[0], "q")
    assert_same(a[1], b[1], "s")


# ---------------------------------------------------------------- weights

def test_quant_weight_linear_small_and_golden():
    d = synth.linear_small()
    q, s = jet.quantize_weight_128x128(bf16_dev(d["w"]))
    qo, so = oracle.quant_weight_128x128(d["w"])
    assert_same(host(q), qo, "qw")
    assert_same(host(s), so, "sw")
    for c in golden_io.quant_cases():
        blk = np.zeros((128, 128), np.float32)
        cols = (np.arange(128) * 37) % 128
        blk[np.arange(128), cols] = np.array(c["x"], np.float32)
        q, s = jet.quantize_weight_128x128(bf16_dev(synth.f32_to_bf16_bits(blk)))
        assert host(s)[0, 0] == np.float32(c["S"]), c["name"]
        want = np.zeros((128, 128), np.uint8)
        want[np.arange(128), cols] = np.array(c["q"], np.uint8)
        assert np.array_equal(host(q), want), c["name"]


@pytest.mark.parametrize("which", ["linear_8b_up", "decode_qkv", "decode_down"])
def test_quant_weight_large_sampled_blocks(which):
    if which == "linear_8b_up":
        w = synth.linear_8b_up()["w"]
    else:
        d = synth.decode_8b(16)
        w = d["w_qkv"] if which == "decode_qkv" else d["w_down"]
    q, s = jet.quantize_weight_128x128(bf16_dev(w))
    q, s = host(q), host(s)
    nb, kb = w.shape[0] // 128, w.shape[1] // 128
    rng = np.random.default_rng(1)
    for _ in range(48):
        i, j = int(rng.integers(nb)), int(rng.integers(kb))
        blk = w[128 * i:128 * i + 128, 128 * j:128 * j + 128]
        qo, so = oracle.quant_weight_128x128(blk)
        assert s[i, j].view(np.uint32) == so[0, 0].view(np.uint32), (i, j)
        assert np.array_equal(q[128 * i:128 * i + 128, 128 * j:128 * j + 128], qo), (i, j)


# ---------------------------------------------------------------- RMSNorm + quant

@pytest.mark.parametrize("m", [16, 64, 256])
def test_rmsnorm_quant_decode_shapes(m):
    d = synth.decode_8b(m)
    q, s = jet.rmsnorm_quant(bf16_dev(d["x"]), bf16_dev(d["gamma"]), d["eps"])
    qo, so = oracle.rmsnorm_quant(d["x"], d["gamma"], d["eps"])
    assert_same(host(q), qo, "q")
    assert_same(host(s), so, "s")


@pytest.mark.parametrize("m,k", [(8195, 4096), (8192, 2048), (2049, 4096), (3000, 8192)])
def test_rmsnorm_quant_training_batches_sampled(m, k):
    """Training-size batches (8k rows, the bench shape and a ragged one; 2049 and 3000
    rows, which split unevenly over the eight XCDs' row ranges of the 2048-workgroup
    grid): bit-exact against the oracle on sampled rows -- the first and last 64,
    rows around the middle, and random rows (rows are independent)."""
    rng = np.random.default_rng(m + k)
    x = synth.random_bf16((m, k), seed=m + k, std=1.0)
    g = synth.f32_to_bf16_bits((1 + 0.05 * rng.standard_normal(k)).astype(np.float32))
    q, s = jet.rmsnorm_quant(bf16_dev(x), bf16_dev(g), 1e-6)
    qh, sh = host(q), host(s)
    half = (m + 1) // 2
    rows = np.unique(np.concatenate([np.arange(64), np.arange(m - 64, m), np.arange(half - 8, half + 8),
                                     rng.integers(0, m, 64)]))
    qo, so = oracle.rmsnorm_quant(x[rows], g, 1e-6)
    assert_same(qh[rows], qo, "q")
    assert_same(sh[:, rows], so, "s")


@pytest.mark.parametrize("m,k", [(1, 128), (5, 640), (3, 2048), (9, 4096), (7, 5120), (3, 7808), (4, 8192),
                                 (2, 12288), (2, 65536)])
def test_rmsnorm_quant_widths(m, k):
    xb = special_rows(m, k, seed=k)
    if m > 1:
        xb[-1] = 0  # an all-zero row: y = 0, S = 1
    rng = np.random.default_rng(k)
    g = synth.f32_to_bf16_bits((1 + 0.05 * rng.standard_normal(k)).astype(np.float32))
    q, s = jet.rmsnorm_quant(bf16_dev(xb), bf16_dev(g), 1e-6)
    qo, so = oracle.rmsnorm_quant(xb, g, 1e-6)
    assert_same(host(q), qo, "q")
    assert_same(host(s), so, "s")


# ---------------------------------------------------------------- requant 1x128 -> 128x1

def requant_gpu(q, s):
    qt, st = jet.requant_transpose_128x1(u8_dev(q), f32_dev(s))
    return host(qt), host(st)


@pytest.mark.parametrize("m,k", [(128, 128), (256, 512), (384, 1024)])
def test_requant_random_codes(m, k):
    rng = np.random.default_rng(m + k)
    q = rng.integers(0, 256, size=(m, k)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    s = (rng.uniform(0.5, 2, size=(k // 128, m)) * np.exp2(rng.integers(-30, 30, size=(k // 128, m)))).astype(np.float32)
    s[0, :3] = 1.0
    q[:, 0] = 0x80  # a column of -0 codes: amax 0 -> S' = 1
    qt, st = requant_gpu(q, s)
    qto, sto = oracle.requant_transpose_128x1(q, s)
    assert_same(qt, qto, "qt")
    assert_same(st, sto, "st")


def test_requant_pipeline_linear_8b_up():
    d = synth.linear_8b_up()
    for name in ("x", "dy"):
        xb = d[name]
        qd, sd = jet.quantize_act_1x128(bf16_dev(xb))
        qt, st = jet.requant_transpose_128x1(qd, sd)
        qt, st = host(qt), host(st)
        rng = np.random.default_rng(2)
        for mb in rng.choice(xb.shape[0] // 128, 4, replace=False):
            rows = slice(128 * mb, 128 * mb + 128)
            qo, so = oracle.quant_act_1x128(xb[rows])
            qto, sto = oracle.requant_transpose_128x1(qo, so)
            assert_same(qt[:, rows], qto, f"{name} qt block {mb}")
            assert_same(st[mb], sto[0], f"{name} st block {mb}")


def test_requant_underflowing_scale():
    """A column whose amax / 448 underflows to zero takes S' = 1 (hand-derived case)."""
    from test_oracle_quant import underflow_scale_case
    q, s, want_qt, want_st = underflow_scale_case()
    qt, st = requant_gpu(q, s)
    assert np.array_equal(qt, want_qt)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


def test_requant_guards():
    rng = np.random.default_rng(9)
    q = rng.integers(0, 0x7E, size=(256, 256)).astype(np.uint8)
    s = rng.uniform(0.1, 1, size=(2, 256)).astype(np.float32)
    qg, sg = Guarded((256, 256), torch.uint8), Guarded((2, 256), torch.float32)
    jet.requant_transpose_128x1(u8_dev(q), f32_dev(s), qg.t, sg.t)
    torch.cuda.synchronize()
    assert qg.intact() and sg.intact()
    qto, sto = oracle.requant_transpose_128x1(q, s)
    assert_same(host(qg.t), qto, "qt")
