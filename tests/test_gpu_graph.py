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


def test_packed_rollout_fused_swiglu_and_split_round_replay_equal_eager():
    """More launch sequences under capture: pack_weight_rollout and the packed FProp at
    16 and 100 tokens (the decode and weight-sharing kernels), the gate+up FProp whose
    epilogue applies SwiGLU and the quantisation (its SiLU table copied into LDS with
    direct loads), and a WGrad with 384 tiles of 256 x 256, whose last half-round runs as
    a second launch on the 128 x 128 kernel.  Every replay, with eager work between,
    equals the eager results bit for bit."""
    dev = torch.device("cuda:0")
    k, n = 512, 768
    x16 = jet.quantize_act_1x128(bf16_dev(synth.random_bf16((16, k), seed=51)))
    x100 = jet.quantize_act_1x128(bf16_dev(synth.random_bf16((100, k), seed=52)))
    qw, sw = jet.quantize_weight_128x128(bf16_dev(synth.random_bf16((n, k), seed=53, std=0.02)))
    mg, ng, kg = 512, 2048, 256  # gate+up: I = 1024
    xg = jet.quantize_act_1x128(bf16_dev(synth.random_bf16((mg, kg), seed=54)))
    wg = jet.quantize_weight_128x128(bf16_dev(synth.random_bf16((ng, kg), seed=55, std=0.02)))
    tok, rows, cols = 256, 6144, 4096  # WGrad: dW [6144][4096] over 256 tokens
    dyt = jet.quantize_act_1x128(bf16_dev(synth.random_bf16((rows, tok), seed=56, std=1e-3)))
    xt = jet.quantize_act_1x128(bf16_dev(synth.random_bf16((cols, tok), seed=57)))
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    qwp = torch.empty(n, k, dtype=u8, device=dev)
    y16, y100 = torch.empty(16, n, dtype=bf, device=dev), torch.empty(100, n, dtype=bf, device=dev)
    qh, sh = torch.empty(mg, ng // 2, dtype=u8, device=dev), torch.empty(ng // 256, mg, dtype=f32, device=dev)
    dw = torch.empty(rows, cols, dtype=bf, device=dev)

    def step():
        jet.pack_weight_rollout(qw, qwp)
        jet.gemm_fprop_packed(*x16, qwp, sw, y16)
        jet.gemm_fprop_packed(*x100, qwp, sw, y100)
        jet.gemm_fprop_swiglu_quant(*xg, *wg, qh, sh)
        jet.gemm_wgrad(*dyt, *xt, dw)

    outs = (qwp, y16, y100, qh, sh, dw)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
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
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}, output {i}"
        step()  # eager work between replays
        torch.cuda.synchronize()
