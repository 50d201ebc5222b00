"""Seeded input generators: determinism, shapes, value structure, bf16 rounding."""

import numpy as np
import torch

from quantized_rl_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), want)


def _f32(u):
    return (u.astype(np.uint32) << 16).view(np.float32)


def test_linear_small_is_deterministic_and_shaped():
    a, b = synth.linear_small(), synth.linear_small()
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["w"], b["w"])
    assert a["x"].shape == (256, 512) and a["w"].shape == (384, 512)
    assert a["x"].dtype == np.uint16
    x = _f32(a["x"])
    ch = a["outlier_channels"]
    assert len(ch) == 2
    colstd = x.std(axis=0)
    assert np.all(colstd[ch] > 30) and np.median(colstd) < 1.2
    assert abs(_f32(a["w"]).std() - 0.02) < 0.002
    assert not np.array_equal(synth.linear_small(seed=5)["x"], a["x"])


def test_decode_and_llama_shapes():
    d = synth.decode_8b(16)
    assert d["x"].shape == (16, 4096) and d["gamma"].shape == (4096,)
    assert d["w_qkv"].shape == (6144, 4096) and d["w_down"].shape == (4096, 12288)
    g = _f32(d["gamma"])
    assert abs(g.mean() - 1.0) < 0.01 and abs(g.std() - 0.05) < 0.01
    ll = synth.llama_layer(0, "down", m=256)
    assert ll["x"].shape == (256, 14336) and ll["w"].shape == (4096, 14336) and ll["dy"].shape == (256, 4096)
    assert len(ll["outlier_channels"]) == 14
    assert abs(_f32(ll["dy"]).std() - 1e-3) < 1e-4
