"""The entry points under HIP graph capture: a whole fwd+bwd step of the FP8
linear (norm+quant, weight quant, FProp, dY quant, DGrad, two requants, WGrad,
fp32 WGrad accumulation) recorded once with torch.cuda.graph and replayed.

The library enqueues only kernel launches on the caller's stream (no memset
nodes, no allocation, no host synchronisation), so capture works unchanged.
Every replay, with eager work and synchronisation in between, must equal the
eager results bit for bit."""

import numpy as np
import pytest
import torch

from gpu_common import bf16_dev
import quantized_rl_amd as jet
from quantized_rl_amd import synth

pytestmark = pytest.mark.gpu


def test_step_replays_equal_eager():
    m, k, n = 4096, 512, 4608  # FProp: 288 tiles of 256 x 256 (the tile loop)
    dev = torch.device("cuda:0")
    x = bf16_dev(synth.random_bf16((m, k), seed=31))
    g = bf16_dev(synth.random_bf16((k,), seed=32, std=0.05)) + 1
    w = bf16_dev(synth.random_bf16((n, k), seed=33, std=0.02))
    dy = bf16_dev(synth.random_bf16((m, n), seed=34, std=1e-3))
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    E = lambda *s, dt: torch.empty(s, dtype=dt, device=dev)
    qx, sx, r = E(m, k, dt=u8), E(k // 128, m, dt=f32), E(m, dt=f32)
    qw, sw = E(n, k, dt=u8), E(n // 128, k // 128, dt=f32)
    qdy, sdy = E(m, n, dt=u8), E(n // 128, m, dt=f32)
    qxt, sxt = E(k, m, dt=u8), E(m // 128, k, dt=f32)
    qdyt, sdyt = E(n, m, dt=u8), E(m // 128, n, dt=f32)
    y, dx, dw = E(m, n, dt=bf), E(m, k, dt=bf), E(n, k, dt=bf)
    dw32 = torch.zeros(n, k, dtype=f32, device=dev)

    def step():
        jet.rmsnorm_quant_rstd(x, g, 1e-6, qx, sx, r)
        jet.quantize_weight_128x128(w, qw, sw)
        jet.gemm_fprop(qx, sx, qw, sw, y)
        jet.quantize_act_1x128(dy, qdy, sdy)
        jet.gemm_dgrad(qdy, sdy, qw, sw, dx)
        jet.requant_transpose_128x1(qx, sx, qxt, sxt)
        jet.requant_transpose_128x1(qdy, sdy, qdyt, sdyt)
        jet.gemm_wgrad(qdyt, sdyt, qxt, sxt, dw)
        jet.gemm_wgrad_f32(qdyt, sdyt, qxt, sxt, dw=dw32, accumulate=True)

    outs = (y, dx, dw, qxt, qdyt, r)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g1 = dw32.clone()  # one accumulated WGrad
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.zero_()
        dw32.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {rep}"
        assert torch.equal(dw32, g1), f"replay {rep}: fp32 accumulation"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(dw32, g1 + g1)


def test_rollout_step_with_split_k_replays_equal_eager():
    """The rollout forward at a 64-token batch through gemm_fprop_splitk (K split
    into shares with fp32 partials in a workspace, then the reduction: two launches
    per projection, no memset) captured once and replayed with eager work in
    between; every replay equals the eager result bit for bit."""
    m, k, n_qkv, n_down, k_down = 64, 1024, 768, 256, 2048
    dev = torch.device("cuda:0")
    x = bf16_dev(synth.random_bf16((m, k), seed=41))
    g = bf16_dev(synth.random_bf16((k,), seed=42, std=0.05)) + 1
    h = bf16_dev(synth.random_bf16((m, k_down), seed=43))
    wq = jet.quantize_weight_128x128(bf16_dev(synth.random_bf16((n_qkv, k), seed=44, std=0.02)))
    wd = jet.quantize_weight_128x128(bf16_dev(synth.random_bf16((n_down, k_down), seed=45, std=0.02)))
    need = max(jet.gemm_fprop_splitk_workspace_bytes(m, n_qkv, k),
               jet.gemm_fprop_splitk_workspace_bytes(m, n_down, k_down))
    assert jet.gemm_fprop_splitk_workspace_bytes(m, n_qkv, k) > 0
    assert jet.gemm_fprop_splitk_workspace_bytes(m, n_down, k_down) > 0
    ws = torch.empty(need // 4, dtype=torch.float32, device=dev)
    qx, sx = jet.rmsnorm_quant(x, g, 1e-6)
    qh, sh = jet.quantize_act_1x128(h)
    y = torch.empty(m, n_qkv, dtype=torch.bfloat16, device=dev)
    yd = torch.empty(m, n_down, dtype=torch.bfloat16, device=dev)

    def step():
        jet.rmsnorm_quant(x, g, 1e-6, qx, sx)
        jet.gemm_fprop_splitk(qx, sx, *wq, y, ws)
        jet.quantize_act_1x128(h, qh, sh)
        jet.gemm_fprop_splitk(qh, sh, *wd, yd, ws)

    step()
    torch.cuda.synchronize()
    ref = [y.clone(), yd.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()
        yd.zero_()
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]) and torch.equal(yd, ref[1]), f"replay {rep}"
        step()  # eager work between replays
        torch.cuda.synchronize()
