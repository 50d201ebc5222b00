"""Seeded synthetic inputs for the FP8 linear layer (shared by tests, bench and smoke).

Holds no quantisation or GEMM arithmetic: it draws numbers and rounds them to
bf16.  Every tensor is produced on the host with numpy's PCG64 generator from a
``SeedSequence`` per workload, drawn in float32 and rounded to bf16 (nearest
even), so the GPU path and the CPU oracle consume identical bf16 bytes.

Child streams of each workload's ``SeedSequence`` are spawned in one fixed
order: outlier-channel choice, X, W, dY, gamma, down-projection input.  When a
workload needs several tensors of one kind they are drawn one after another
from that kind's stream.  "N(mu, sigma)" means mean mu, standard deviation
sigma.  An outlier channel is a column of X (an input feature).

Workloads (shapes of Qwen3-8B, Llama-3.1-8B and a Qwen3-32B half-MLP; the pages'
own runs used real models and math-RL data that are not reproduced here):

* ``linear_small``  -- X [256, 512] N(0,1) with 2 outlier channels x50,
  W [384, 512] N(0, 0.02).
* ``linear_8b_up``  -- X [8192, 4096] N(0,1) with round(0.1% K) = 4 outlier
  channels x50, W [12288, 4096] N(0, 0.02), dY [8192, 12288] N(0, 1e-3).
* ``decode_8b``     -- X [M, 4096] N(0,1), gamma [4096] N(1, 0.05),
  W_qkv [6144, 4096], W_gu [24576, 4096], W_down [4096, 12288] N(0, 0.02),
  down input [M, 12288] N(0, 1); M in {16, 64, 256}.
* ``llama_layer``   -- one linear of a Llama-3.1-8B layer stack at M = 16384:
  X N(0,1) whose round(0.1% K) outlier channels hold unscaled Student-t(3)
  draws, W N(0, 0.02), dY N(0, 1e-3).
* ``qwen32b_half_mlp`` -- X [M, 5120], W_gu [25600, 5120], W_down [5120, 12800]
  N(0, 0.02), down input [M, 12800] N(0,1); at M = 8192 also dY_gu [M, 25600]
  and dY_down [M, 5120] N(0, 1e-3).
"""

import numpy as np

_KINDS = ("outliers", "x", "w", "dy", "gamma", "down_in")

LLAMA_LINEARS = {  # name: (N, K)
    "qkv": (6144, 4096),
    "o": (4096, 4096),
    "gate_up": (28672, 4096),
    "down": (4096, 14336),
}


def f32_to_bf16_bits(a):
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _streams(seed, key=()):
    ss = np.random.SeedSequence(entropy=seed, spawn_key=tuple(key))
    return dict(zip(_KINDS, (np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(len(_KINDS)))))


def _normal(rng, shape, mean=0.0, std=1.0):
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    if mean != 0.0:
        z += np.float32(mean)
    return z


def _activation(st, m, k, n_out, scale=None, student_t=False):
    ch = np.sort(st["outliers"].choice(k, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    x = _normal(st["x"], (m, k))
    if n_out:
        if student_t:
            x[:, ch] = st["x"].standard_t(3, size=(m, n_out)).astype(np.float32)
        else:
            x[:, ch] *= np.float32(scale)
    return x, ch


def linear_small(seed=0):
    st = _streams(seed)
    x, ch = _activation(st, 256, 512, 2, scale=50.0)
    w = _normal(st["w"], (384, 512), std=0.02)
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w), "outlier_channels": ch}


def linear_8b_up(seed=1, m=8192, n=12288, k=4096):
    st = _streams(seed)
    x, ch = _activation(st, m, k, int(round(0.001 * k)), scale=50.0)
    w = _normal(st["w"], (n, k), std=0.02)
    dy = _normal(st["dy"], (m, n), std=1e-3)
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w), "dy": f32_to_bf16_bits(dy),
            "outlier_channels": ch}


def decode_8b(m, seed=2):
    st = _streams(seed, (m,))
    x = _normal(st["x"], (m, 4096))
    w_qkv = _normal(st["w"], (6144, 4096), std=0.02)
    w_gu = _normal(st["w"], (24576, 4096), std=0.02)
    w_down = _normal(st["w"], (4096, 12288), std=0.02)
    gamma = _normal(st["gamma"], (4096,), mean=1.0, std=0.05)
    h = _normal(st["down_in"], (m, 12288))
    b = f32_to_bf16_bits
    return {"x": b(x), "gamma": b(gamma), "w_qkv": b(w_qkv), "w_gu": b(w_gu), "w_down": b(w_down),
            "down_in": b(h), "eps": 1e-6}


def llama_layer(layer, name, m=16384, seed=3):
    n, k = LLAMA_LINEARS[name]
    st = _streams(seed, (layer, list(LLAMA_LINEARS).index(name)))
    x, ch = _activation(st, m, k, int(round(0.001 * k)), student_t=True)
    w = _normal(st["w"], (n, k), std=0.02)
    dy = _normal(st["dy"], (m, n), std=1e-3)
    return {"x": f32_to_bf16_bits(x), "w": f32_to_bf16_bits(w), "dy": f32_to_bf16_bits(dy),
            "outlier_channels": ch}


def qwen32b_half_mlp(m, seed=4):
    st = _streams(seed, (m,))
    b = f32_to_bf16_bits
    out = {
        "x": b(_normal(st["x"], (m, 5120))),
        "w_gu": b(_normal(st["w"], (25600, 5120), std=0.02)),
        "w_down": b(_normal(st["w"], (5120, 12800), std=0.02)),
        "down_in": b(_normal(st["down_in"], (m, 12800))),
    }
    if m == 8192:
        out["dy_gu"] = b(_normal(st["dy"], (m, 25600), std=1e-3))
        out["dy_down"] = b(_normal(st["dy"], (m, 5120), std=1e-3))
    return out


def random_bf16(shape, seed, std=1.0):
    """Plain N(0, std) bf16 tensor for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return f32_to_bf16_bits(_normal(rng, shape, std=std))
