"""Host-side construction of the FP8 linear module (no kernel is called)."""

import pytest
import torch

from quantized_rl_amd import linear


def test_fp8_linear_module_buffers():
    plain = linear.FP8Linear(256, 128, device="cpu")
    assert plain.main_grad is None
    assert plain.weight.dtype == torch.bfloat16 and tuple(plain.weight.shape) == (128, 256)
    plain.zero_main_grad()  # nothing to clear
    acc = linear.FP8Linear(256, 128, device="cpu", fp32_grad_accum=True)
    assert acc.main_grad.dtype == torch.float32 and tuple(acc.main_grad.shape) == (128, 256)
    assert bool((acc.main_grad == 0).all())
    acc.main_grad.fill_(2.0)
    acc.zero_main_grad()
    assert bool((acc.main_grad == 0).all())
    assert "main_grad" not in acc.state_dict()  # not persistent: the master weight is the state


def test_fp8_linear_module_rejects_unaligned_features():
    with pytest.raises(ValueError):
        linear.FP8Linear(100, 128, device="cpu")
    with pytest.raises(ValueError):
        linear.FP8Linear(128, 200, device="cpu")


def test_rmsnorm_fp8_linear_module_parameters():
    blk = linear.RMSNormFP8Linear(256, 128, eps=1e-5, device="cpu")
    assert blk.gamma.dtype == torch.bfloat16 and bool((blk.gamma == 1).all())
    assert tuple(blk.weight.shape) == (128, 256) and blk.eps == 1e-5
    with pytest.raises(ValueError):
        linear.RMSNormFP8Linear(200, 128, device="cpu")


def test_fp8_stack_shapes():
    st = linear.FP8Stack([512, 1024, 512, 768, 384], device="cpu")
    assert len(st.layers) == 4
    assert [tuple(l.weight.shape) for l in st.layers] == [(1024, 512), (512, 1024), (768, 512), (384, 768)]
    with pytest.raises(ValueError):
        linear.FP8Stack([512], device="cpu")


def test_rmsnorm_fp8_linear_rejects_rows_past_the_backward_limit():
    linear.RMSNormFP8Linear(linear.RMSNORM_BACKWARD_MAX_K, 128, device="meta")
    with pytest.raises(ValueError, match="RMSNorm backward"):
        linear.RMSNormFP8Linear(linear.RMSNORM_BACKWARD_MAX_K + 128, 128, device="meta")


def test_weight_cache_requantises_only_on_change(monkeypatch):
    calls = []

    def fake_quant(w):
        calls.append(w.data_ptr())
        return ("q", len(calls)), ("s", len(calls))

    monkeypatch.setattr(linear._lib, "quantize_weight_128x128", fake_quant)
    w = torch.zeros(128, 256, dtype=torch.bfloat16)
    c = linear.WeightCache()
    a = c.get(w)
    assert c.get(w) is not None and c.get(w) == a and c.quantizations == 1   # unchanged: reused
    with torch.no_grad():
        w.add_(1)                                                              # in-place update
    b = c.get(w)
    assert b != a and c.quantizations == 2
    w2 = w.clone()                                                             # another tensor
    c.get(w2)
    assert c.quantizations == 3 and calls[-1] == w2.data_ptr()


def test_rollout_path_rule():
    """The rollout path is taken only when no autograd graph is needed and the batch
    fits gemm_fprop_packed (at most 256 rows)."""
    w = torch.zeros(256, 512, dtype=torch.bfloat16, requires_grad=True)
    x = torch.zeros(16, 512, dtype=torch.bfloat16)
    assert not linear.rollout_path(x, w)                   # the weight needs a gradient
    with torch.no_grad():
        assert linear.rollout_path(x, w)
        assert linear.rollout_path(torch.zeros(256, 512, dtype=torch.bfloat16), w)
        assert not linear.rollout_path(torch.zeros(257, 512, dtype=torch.bfloat16), w)
    w_frozen = w.detach()
    assert linear.rollout_path(x, w_frozen)                # frozen weight, plain input
    assert not linear.rollout_path(x.clone().requires_grad_(), w_frozen)


def test_weight_cache_packs_once_per_version(monkeypatch):
    packs = []
    monkeypatch.setattr(linear._lib, "quantize_weight_128x128", lambda w: (("q", w._version), "s"))
    monkeypatch.setattr(linear._lib, "pack_weight_rollout", lambda q: packs.append(q) or ("p", q))
    w = torch.zeros(128, 256, dtype=torch.bfloat16)
    c = linear.WeightCache()
    a = c.get_packed(w)
    assert c.get_packed(w) == a and c.packs == 1 and c.quantizations == 1
    with torch.no_grad():
        w.add_(1)
    b = c.get_packed(w)
    assert b != a and c.packs == 2 and c.quantizations == 2
    c.get(w)                                               # the FP8 form alone: no new pack
    assert c.packs == 2
