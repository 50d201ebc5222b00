"""GPU parity of swiglu_quant (SiLU(gate) * up, quantised 1x128) with the oracle,
bit for bit: codes and scales.

The gate values are bf16, so silu has 65536 possible arguments: every one of
them is run (i) next to random up values and (ii) as a whole group of 128 equal
elements with up = 1, where the group's scale S = fl32(|silu(g)| / 448) moves
with silu's last bits.  Plus the hand-derived golden groups, ragged and model
shapes (the Qwen3-8B and Llama-3.1-8B intermediate sizes, the Qwen3-32B half
MLP's), sampled rows of a training batch, guards and determinism.
"""

import numpy as np
import pytest
import torch

import golden_io
import oracle
from gpu_common import Guarded, bf16_dev, host
import quantized_rl_amd as jet
from quantized_rl_amd import synth
from quantized_rl_amd.synth import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def finite_bf16_bits():
    u = np.arange(1 << 16, dtype=np.uint32)
    v = (u << 16).view(np.float32)
    return u[np.isfinite(v)].astype(np.uint16)


def run(y):
    q, s = jet.swiglu_quant(bf16_dev(y))
    return host(q), host(s)


def check_bits(y, what):
    print(f"[swiglu_quant] {what} y={y.shape}", flush=True)
    q, s = run(y)
    qo, so = oracle.swiglu_quant(y)
    assert np.array_equal(q, qo), f"{what}: codes differ at {np.argwhere(q != qo)[:5]}"
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), f"{what}: scales differ"


def test_every_gate_value_with_random_up():
    g = finite_bf16_bits()
    rng = np.random.default_rng(1)
    g = g[rng.permutation(g.size)]
    i = 1024
    m = (g.size + i - 1) // i
    gate = np.zeros(m * i, np.uint16)
    gate[:g.size] = g
    # |up| <= 1 keeps h = silu(g) * up finite next to the largest gates
    up = f32_to_bf16_bits(rng.uniform(-1.0, 1.0, size=(m, i)).astype(np.float32))
    check_bits(np.concatenate([gate.reshape(m, i), up], axis=1), "every gate, random up")


def test_every_gate_value_as_a_uniform_group():
    g = finite_bf16_bits()
    i = 128 * 128
    m = (g.size + 127) // 128
    gate = np.zeros((m * 128, 128), np.uint16)
    gate[:g.size] = g[:, None]
    gate = gate.reshape(m, i)
    one = np.full((m, i), 0x3F80, np.uint16)  # bf16 1.0
    check_bits(np.concatenate([gate, one], axis=1), "every gate, uniform groups")


def _exact_over_32(case):
    """The hand-derived group can be placed as h = silu(32) * (x / 32) only where x / 32
    is exact in bf16 (the subnormal-scale case is not)."""
    x = np.array(case["x"], np.float32)
    return np.array_equal(oracle.bf16_bits_to_f32(f32_to_bf16_bits(x / np.float32(32))) * np.float32(32), x)


@pytest.mark.parametrize("case", [c for c in golden_io.quant_cases() if _exact_over_32(c)], ids=lambda c: c["name"])
def test_golden_group(case):
    x = np.array(case["x"], np.float32)
    m, i = 3, 512
    gate = np.full((m, i), -100.0, np.float32)
    up = np.ones((m, i), np.float32)
    gate[1, 256:384] = 32.0
    up[1, 256:384] = x / np.float32(32)
    y = f32_to_bf16_bits(np.concatenate([gate, up], axis=1))
    q, s = run(y)
    assert s[2, 1] == np.float32(case["S"])
    assert np.array_equal(q[1, 256:384], np.array(case["q"], np.uint8))
    check_bits(y, f"golden {case['name']}")


# 4-row tiles up to 128 rows, 8-row tiles up to 512, 32-row tiles above (ragged in each)
@pytest.mark.parametrize("m,i", [(1, 128), (33, 384), (64, 640), (100, 1152), (257, 512), (2, 12288),
                                 (16, 14336), (65, 12800), (256, 12288), (300, 384), (520, 640)])
def test_shapes(m, i):
    y = synth.random_bf16((m, 2 * i), seed=m + i, std=3.0)
    check_bits(y, f"{m}x{i}")


def test_training_batch_sampled_rows():
    """8192 tokens of the Qwen3-8B MLP (I = 12288): the whole batch on the GPU,
    the oracle on 64 sampled rows (rows are independent)."""
    m, i = 8192, 12288
    y = synth.random_bf16((m, 2 * i), seed=9, std=2.0)
    q, s = run(y)
    rows = np.sort(np.random.default_rng(3).choice(m, 64, replace=False))
    qo, so = oracle.swiglu_quant(y[rows])
    assert np.array_equal(q[rows], qo)
    assert np.array_equal(s[:, rows].view(np.uint32), so.view(np.uint32))


def test_guards_empty_and_determinism():
    m, i = 96, 640
    y = synth.random_bf16((m, 2 * i), seed=4)
    qg, sg = Guarded((m, i), torch.uint8), Guarded((i // 128, m), torch.float32)
    jet.swiglu_quant(bf16_dev(y), qg.t, sg.t)
    torch.cuda.synchronize()
    assert qg.intact() and sg.intact()
    q2, s2 = run(y)
    assert np.array_equal(host(qg.t), q2) and np.array_equal(host(sg.t), s2)
    q0, s0 = jet.swiglu_quant(torch.empty((0, 2 * i), dtype=torch.bfloat16, device="cuda:0"))
    assert q0.shape == (0, i) and s0.shape == (i // 128, 0)
