"""The FP8 linear autograd op (quantized_rl_amd.linear) on the GPU.

Its forward and backward must be exactly the C-ABI pipeline: the gradients
torch's autograd returns are checked against the oracle's pipeline on the same
bf16 inputs (quantisers bit-exact upstream, GEMMs to the GEMM tolerance), the
tensors saved for backward are the FP8 codes and scales, and a two-layer stack
trains through autograd.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import bf16_dev, host
from quantized_rl_amd import _lib, linear, synth

pytestmark = pytest.mark.gpu


def check(y, ref, what):
    r = oracle.check_gemm(y, ref)
    assert r["ok"], f"{what}: {r}"


@pytest.mark.parametrize("m,k,n", [(256, 512, 384), (384, 640, 256)])
def test_fp8_linear_autograd_matches_the_oracle_pipeline(m, k, n):
    x_h = synth.random_bf16((m, k), seed=m + k, std=1.0)
    w_h = synth.random_bf16((n, k), seed=n + 1, std=0.02)
    dy_h = synth.random_bf16((m, n), seed=m + n, std=1e-3)
    x = bf16_dev(x_h).requires_grad_(True)
    w = bf16_dev(w_h).requires_grad_(True)
    y = linear.fp8_linear(x, w)
    y.backward(bf16_dev(dy_h))
    torch.cuda.synchronize()

    qxo, sxo = oracle.quant_act_1x128(x_h)
    qwo, swo = oracle.quant_weight_128x128(w_h)
    qdyo, sdyo = oracle.quant_act_1x128(dy_h)
    check(host(y.detach()), oracle.gemm_fprop_ref(qxo, sxo, qwo, swo), "y")
    check(host(x.grad), oracle.gemm_dgrad_ref(qdyo, sdyo, qwo, swo), "dx")
    qxt, sxt = oracle.requant_transpose_128x1(qxo, sxo)
    qdyt, sdyt = oracle.requant_transpose_128x1(qdyo, sdyo)
    check(host(w.grad), oracle.gemm_wgrad_ref(qdyt, sdyt, qxt, sxt), "dw")


def test_fp8_linear_saves_fp8_activations_only():
    m, k, n = 256, 512, 384
    x = bf16_dev(synth.random_bf16((m, k), seed=5)).requires_grad_(True)
    w = bf16_dev(synth.random_bf16((n, k), seed=6, std=0.02)).requires_grad_(True)
    saved = []
    with torch.autograd.graph.saved_tensors_hooks(lambda t: saved.append(t) or t, lambda t: t):
        y = linear.fp8_linear(x, w)
    assert sorted(str(t.dtype) for t in saved) == ["torch.float32", "torch.float32", "torch.uint8", "torch.uint8"]
    assert any(t.dtype == torch.uint8 and tuple(t.shape) == (m, k) for t in saved)  # FP8 X, no bf16 copy
    y.sum().backward()


def test_fp8_linear_rejects_ragged_tokens_in_backward():
    x = bf16_dev(synth.random_bf16((100, 256), seed=7)).requires_grad_(True)
    w = bf16_dev(synth.random_bf16((128, 256), seed=8, std=0.02)).requires_grad_(True)
    y = linear.fp8_linear(x, w)  # the forward accepts any M
    with pytest.raises(ValueError):
        y.backward(torch.ones_like(y))


def test_two_layer_fp8_stack_trains():
    """Two FP8Linear layers: one SGD step on a least-squares loss lowers the loss,
    and each layer's gradients equal the functional op applied to the same tensors."""
    torch.manual_seed(0)
    dev = torch.device("cuda:0")
    l1, l2 = linear.FP8Linear(512, 384, device=dev), linear.FP8Linear(384, 256, device=dev)
    x = torch.randn(256, 512, device=dev).to(torch.bfloat16)
    target = torch.randn(256, 256, device=dev).to(torch.bfloat16) * 0.01

    def loss_fn():
        return ((l2(l1(x)).float() - target.float()) ** 2).mean()

    loss0 = loss_fn()
    loss0.backward()
    g1, g2 = l1.weight.grad.clone(), l2.weight.grad.clone()
    assert torch.isfinite(g1.float()).all() and torch.isfinite(g2.float()).all()
    # the same gradients from the functional op on the same tensors
    h = linear.fp8_linear(x, l1.weight.detach())
    h_req = h.detach().requires_grad_(True)
    w2 = l2.weight.detach().clone().requires_grad_(True)
    out = linear.fp8_linear(h_req, w2)
    ((out.float() - target.float()) ** 2).mean().backward()
    assert torch.equal(w2.grad, g2)
    with torch.no_grad():
        for p in (l1.weight, l2.weight):
            p -= (5.0 * p.grad.float()).to(torch.bfloat16)
            p.grad = None
    assert loss_fn().item() < loss0.item()


def test_fp8_linear_fp32_grad_accumulation_over_micro_batches():
    """FP8Linear(fp32_grad_accum=True): two micro-batches add their weight
    gradients into main_grad in fp32 (no gradient lands in weight.grad); the sum
    equals the two fp32 WGrad results added in fp32, each of which rounds to the
    bf16 gradient of the plain layer, and it matches the oracle's fp64 sum."""
    torch.manual_seed(1)
    dev = torch.device("cuda:0")
    m, k, n = 256, 512, 384
    layer = linear.FP8Linear(k, n, device=dev, fp32_grad_accum=True)
    w = layer.weight.detach().clone()
    xs = [synth.random_bf16((m, k), seed=40 + i, std=1.0) for i in range(2)]
    dys = [synth.random_bf16((m, n), seed=50 + i, std=1e-3) for i in range(2)]
    parts = []
    for x_h, dy_h in zip(xs, dys):
        x = bf16_dev(x_h).requires_grad_(True)
        layer(x).backward(bf16_dev(dy_h))
        # the same micro-batch through the plain bf16 path and through gemm_wgrad_f32
        x2 = bf16_dev(x_h).requires_grad_(True)
        w2 = w.clone().requires_grad_(True)
        linear.fp8_linear(x2, w2).backward(bf16_dev(dy_h))
        qx, sx = jet_quant(x2)
        qdy, sdy = jet_quant(bf16_dev(dy_h))
        qxt, sxt = _lib.requant_transpose_128x1(qx, sx)
        qdyt, sdyt = _lib.requant_transpose_128x1(qdy, sdy)
        g = host(_lib.gemm_wgrad_f32(qdyt, sdyt, qxt, sxt))
        assert np.array_equal(host(w2.grad), oracle.f64_to_bf16_bits(g.astype(np.float64)))
        assert torch.equal(x.grad, x2.grad)
        parts.append(g)
    torch.cuda.synchronize()
    assert layer.weight.grad is None
    assert np.array_equal(host(layer.main_grad), np.float32(0) + parts[0] + parts[1])
    ref = 0.0
    for x_h, dy_h in zip(xs, dys):
        qxo, sxo = oracle.quant_act_1x128(x_h)
        qdyo, sdyo = oracle.quant_act_1x128(dy_h)
        qxt, sxt = oracle.requant_transpose_128x1(qxo, sxo)
        qdyt, sdyt = oracle.requant_transpose_128x1(qdyo, sdyo)
        ref = ref + oracle.gemm_wgrad_ref(qdyt, sdyt, qxt, sxt)
    r = oracle.check_gemm_f32(host(layer.main_grad), ref)
    assert r["ok"], r
    layer.zero_main_grad()
    assert bool((layer.main_grad == 0).all())


def jet_quant(t):
    return _lib.quantize_act_1x128(t.detach().contiguous())


def test_four_layer_fp8_stack_trains_and_chains_the_layers():
    """FP8Stack of four RMSNorm+FP8 linear layers: the input gradient equals the
    layers' backward applied one after the other (each through its own autograd
    op on the same tensors), and two SGD steps on a least-squares loss lower it."""
    torch.manual_seed(4)
    dev = torch.device("cuda:0")
    stack = linear.FP8Stack([512, 1024, 512, 768, 384], device=dev)
    x = bf16_dev(synth.random_bf16((256, 512), seed=61)).requires_grad_(True)
    target = torch.randn(256, 384, device=dev).to(torch.bfloat16) * 0.01

    def loss_of(y):
        return ((y.float() - target.float()) ** 2).mean()

    y = stack(x)
    loss0 = loss_of(y)
    (gy,) = torch.autograd.grad(loss0, y, retain_graph=True)
    loss0.backward()
    gx = x.grad.clone()
    # the same chain, layer by layer, on detached activations
    acts = [x.detach()]
    for layer in stack.layers:
        acts.append(layer(acts[-1]).detach())
    assert torch.equal(acts[-1], y.detach())
    grad = gy
    for layer, a in zip(reversed(stack.layers), reversed(acts[:-1])):
        a = a.clone().requires_grad_(True)
        layer(a).backward(grad)
        grad = a.grad
    assert torch.equal(grad, gx)
    for _ in range(2):
        stack.zero_grad(set_to_none=True)
        loss_of(stack(x.detach())).backward()
        with torch.no_grad():
            for p in stack.parameters():
                p -= (2.0 * p.grad.float()).to(p.dtype)
    assert loss_of(stack(x.detach())).item() < loss0.item()


def test_weight_quantised_once_per_update(monkeypatch):
    """Two forwards with no weight update launch one weight quantisation and give
    bitwise-equal outputs; an optimizer step (in place) triggers a new one, whose
    codes equal a fresh quantisation of the updated weight."""
    calls = []
    real = _lib.quantize_weight_128x128

    def counting(w, *a, **kw):
        calls.append(1)
        return real(w, *a, **kw)

    monkeypatch.setattr(_lib, "quantize_weight_128x128", counting)
    torch.manual_seed(3)
    for mod in (linear.FP8Linear(512, 384, device="cuda:0"), linear.RMSNormFP8Linear(512, 384, device="cuda:0")):
        calls.clear()
        x = torch.randn(256, 512, device="cuda:0").to(torch.bfloat16)
        y1 = mod(x)
        y2 = mod(x)
        torch.cuda.synchronize()
        assert len(calls) == 1
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        y2.float().sum().backward()
        torch.optim.SGD(mod.parameters(), lr=10.0).step()
        y3 = mod(x)
        torch.cuda.synchronize()
        assert len(calls) == 2 and not torch.equal(y3.view(torch.int16), y1.view(torch.int16))
        qw, sw = real(mod.weight.detach().contiguous())
        assert torch.equal(mod.wcache.q, qw) and torch.equal(mod.wcache.s.view(torch.int32), sw.view(torch.int32))


@pytest.mark.parametrize("m", [1, 16, 40, 64, 65, 200, 256, 257])
def test_rollout_forward_equals_training_forward(m):
    """Without autograd a forward of at most 256 rows runs gemm_fprop_packed on the
    cached packed weight: its output is bitwise the training forward's, the weight is
    packed once per version, and 257 rows take the ordinary path (no pack)."""
    torch.manual_seed(11 + m)
    for mod in (linear.FP8Linear(512, 384, device="cuda:0"), linear.RMSNormFP8Linear(512, 384, device="cuda:0")):
        x = torch.randn(m, 512, device="cuda:0").to(torch.bfloat16)
        y_train = mod(x)                                    # autograd graph: the training forward
        with torch.no_grad():
            y_roll = mod(x)
            y_roll2 = mod(x)
        torch.cuda.synchronize()
        assert torch.equal(y_roll.view(torch.int16), y_train.detach().view(torch.int16)), (type(mod).__name__, m)
        assert torch.equal(y_roll2.view(torch.int16), y_roll.view(torch.int16))
        assert mod.wcache.packs == (1 if m <= 256 else 0) and mod.wcache.quantizations == 1
        with torch.no_grad():
            mod.weight.mul_(0.5)                            # a weight update: new FP8 form and packed copy
            y_half = mod(x)
        torch.cuda.synchronize()
        assert mod.wcache.quantizations == 2 and mod.wcache.packs == (2 if m <= 256 else 0)
        assert not torch.equal(y_half.view(torch.int16), y_roll.view(torch.int16))
