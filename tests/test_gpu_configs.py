"""GPU parity at the full sizes of every workload (sampled outputs vs the oracle).

Workloads (seeded synthetic inputs, see quantized_rl_amd/synth.py):
  linear_small      X [256, 512], W [384, 512]                      FProp
  linear_8b_up      Qwen3-8B up-projection, M=8192                  fwd+bwd (test_gpu_gemm.py)
  decode_8b         M in {16, 64, 256}: RMSNorm+quant, QKV / gate+up / down FProp
  llama_layer       Llama-3.1-8B QKV, O, gate+up, down at M=16384   fwd+bwd
  qwen32b_half_mlp  one GPU's half of a Qwen3-32B MLP               M=256 FProp, M=8192 fwd+bwd
Quantised bytes are checked bit for bit on sampled rows / blocks; GEMM outputs
on sampled (row, column) grids to the normwise / elementwise tolerance.
"""

import numpy as np
import pytest

import oracle
from gpu_common import (act_rows_deq, bf16_dev, check_sampled, host, linear_fwd_bwd_check,
                        weight_rows_deq)
import quantized_rl_amd as jet
from quantized_rl_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m", [16, 64, 256])
def test_decode_8b(m):
    d = synth.decode_8b(m)
    eps = d["eps"]
    print(f"[decode_8b] M={m}", flush=True)
    qx, sx = jet.rmsnorm_quant(bf16_dev(d["x"]), bf16_dev(d["gamma"]), eps)
    qxo, sxo = oracle.rmsnorm_quant(d["x"], d["gamma"], eps)
    assert np.array_equal(host(qx), qxo) and np.array_equal(host(sx).view(np.uint32), sxo.view(np.uint32))
    xdeq = oracle.dequant_groups(qxo, sxo)
    rng = np.random.default_rng(m)
    for name in ("w_qkv", "w_gu"):
        w = d[name]
        qw, sw = jet.quantize_weight_128x128(bf16_dev(w))
        y = host(jet.gemm_fprop(qx, sx, qw, sw))
        cols = np.sort(rng.choice(w.shape[0], 96, replace=False))
        check_sampled(y[:, cols], xdeq @ weight_rows_deq(w, cols).T, f"decode {name} M={m}")
    # down projection: 1x128 quantisation of the [M, 12288] input
    h = d["down_in"]
    qh, sh = jet.quantize_act_1x128(bf16_dev(h))
    qho, sho = oracle.quant_act_1x128(h)
    assert np.array_equal(host(qh), qho) and np.array_equal(host(sh).view(np.uint32), sho.view(np.uint32))
    qw, sw = jet.quantize_weight_128x128(bf16_dev(d["w_down"]))
    y = host(jet.gemm_fprop(qh, sh, qw, sw))
    cols = np.sort(rng.choice(4096, 96, replace=False))
    check_sampled(y[:, cols], oracle.dequant_groups(qho, sho) @ weight_rows_deq(d["w_down"], cols).T,
                  f"decode down M={m}")


@pytest.mark.parametrize("m", [16, 64, 256])
def test_unified_flow_rollout_rows_inside_training_batch(m):
    """The unified precision flow at kernel level: the rollout graph is a
    subgraph of the training forward.  The decode tokens of the 8B workload,
    normalised+quantised and multiplied by the FP8 QKV weight at rollout shape
    (M = 16: decode kernel; 64 and 256: weight-sharing kernel; over the
    row-major weight and over its rollout-packed copy) and inside an 8192-token
    training batch (256 x 256 kernel), give identical FP8 codes, scales and
    FProp outputs, bit for bit; the rollout side also matches the oracle."""
    d = synth.decode_8b(m)
    eps, r0 = d["eps"], 1000
    big = synth.random_bf16((8192, 4096), seed=77 + m, std=1.0)
    big[r0:r0 + m] = d["x"]
    g_d = bf16_dev(d["gamma"])
    qd, sd = jet.rmsnorm_quant(bf16_dev(d["x"]), g_d, eps)
    qb, sb = jet.rmsnorm_quant(bf16_dev(big), g_d, eps)
    qw, sw = jet.quantize_weight_128x128(bf16_dev(d["w_qkv"]))
    yd = host(jet.gemm_fprop(qd, sd, qw, sw))
    yp = host(jet.gemm_fprop_packed(qd, sd, jet.pack_weight_rollout(qw), sw))
    yb = host(jet.gemm_fprop(qb, sb, qw, sw))[r0:r0 + m]
    qdh, sdh = host(qd), host(sd)
    assert np.array_equal(qdh, host(qb)[r0:r0 + m]), "FP8 codes differ between rollout and training batch"
    assert np.array_equal(sdh.view(np.uint32), host(sb)[:, r0:r0 + m].view(np.uint32)), "scales differ"
    assert np.array_equal(yd, yb), "FProp output differs between rollout and training batch"
    assert np.array_equal(yp, yb), "packed FProp output differs from the training batch"
    qo, so = oracle.rmsnorm_quant(d["x"], d["gamma"], eps)
    assert np.array_equal(qdh, qo) and np.array_equal(sdh.view(np.uint32), so.view(np.uint32))
    cols = np.sort(np.random.default_rng(m).choice(6144, 96, replace=False))
    check_sampled(yd[:, cols], oracle.dequant_groups(qo, so) @ weight_rows_deq(d["w_qkv"], cols).T,
                  f"rollout qkv M={m}")


LLAMA_SAMPLE_SEEDS = {"qkv": 11, "o": 12, "gate_up": 13, "down": 14}


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_llama_layer0(name):
    d = synth.llama_layer(0, name)
    linear_fwd_bwd_check(d["x"], d["w"], d["dy"], f"llama layer0 {name}", seed=LLAMA_SAMPLE_SEEDS[name])


def test_llama_layer3_down():
    d = synth.llama_layer(3, "down")
    linear_fwd_bwd_check(d["x"], d["w"], d["dy"], "llama layer3 down", seed=3)


def test_qwen32b_half_mlp_decode():
    d = synth.qwen32b_half_mlp(256)
    linear_fwd_bwd_check(d["x"], d["w_gu"], None, "qwen32b gate_up M=256", backward=False)
    linear_fwd_bwd_check(d["down_in"], d["w_down"], None, "qwen32b down M=256", backward=False)


def test_qwen32b_half_mlp_train():
    d = synth.qwen32b_half_mlp(8192)
    linear_fwd_bwd_check(d["x"], d["w_gu"], d["dy_gu"], "qwen32b gate_up M=8192", seed=1)
    linear_fwd_bwd_check(d["down_in"], d["w_down"], d["dy_down"], "qwen32b down M=8192", seed=2)


def test_linear_small_full():
    d = synth.linear_small()
    linear_fwd_bwd_check(d["x"], d["w"], None, "linear_small", n_rows=256, n_cols=384, backward=False)
