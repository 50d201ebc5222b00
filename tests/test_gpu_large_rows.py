"""GEMMs whose row operand or output passes 2^31 bytes: the library launches them
as row ranges that fit its kernels' 32-bit byte offsets.  Each result must equal,
bit for bit, the same problem computed as separate calls on a different split of
the rows (each within the offsets), and sampled outputs must meet the oracle's
GEMM acceptance.  The operands are seeded quantised Gaussians made on the GPU
(quantize_act_1x128 / quantize_weight_128x128 of torch.randn); the oracle reads
back only the rows it needs."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import host
import quantized_rl_amd as jet
from test_gpu_gemm import check

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def act(m, k, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return jet.quantize_act_1x128(torch.randn(m, k, device=DEV, generator=g).to(torch.bfloat16))


def weight(n, k, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return jet.quantize_weight_128x128((0.02 * torch.randn(n, k, device=DEV, generator=g)).to(torch.bfloat16))


def rows_of(q, s, r0, r1):
    """Rows r0 .. r1 - 1 of a 1x128-quantised [M][K] tensor (scales [K/128][M])."""
    return q[r0:r1], s[:, r0:r1].contiguous()


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_fprop_output_past_2gib():
    """Y [33024][32768] bf16 = 2.16 GB: two row ranges inside the library; the
    reference splits the rows at 16384 instead."""
    m, n, k, cut = 33024, 32768, 256, 16384
    print(f"[large rows] fprop {m}x{n}x{k}", flush=True)
    qx, sx = act(m, k, 1)
    qw, sw = weight(n, k, 2)
    y = jet.gemm_fprop(qx, sx, qw, sw)
    ya = jet.gemm_fprop(*rows_of(qx, sx, 0, cut), qw, sw)
    assert torch.equal(y[:cut].view(torch.int16), ya.view(torch.int16))
    del ya
    yb = jet.gemm_fprop(*rows_of(qx, sx, cut, m), qw, sw)
    assert torch.equal(y[cut:].view(torch.int16), yb.view(torch.int16))
    del yb
    rng = np.random.default_rng(3)
    rows = np.sort(np.concatenate([rng.choice(m, 6, replace=False), [16639, 16640, m - 1]]))
    cols = np.sort(rng.choice(n, 64, replace=False))
    ref = oracle.gemm_fprop_ref_at(host(qx), host(sx), host(qw), host(sw), rows, cols)
    check(host(y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)]), ref, "fprop past 2 GiB")
    del y
    free()


def test_fprop_quant_output_past_2gib():
    """gemm_fprop_quant at the same size: y as gemm_fprop, (qy, sy) equal to
    quantize_act_1x128(y)."""
    m, n, k = 33024, 32768, 256
    print(f"[large rows] fprop_quant {m}x{n}x{k}", flush=True)
    qx, sx = act(m, k, 1)
    qw, sw = weight(n, k, 2)
    y, qy, sy = jet.gemm_fprop_quant(qx, sx, qw, sw)
    y2 = jet.gemm_fprop(qx, sx, qw, sw)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    del y2
    q2, s2 = jet.quantize_act_1x128(y)
    assert torch.equal(qy, q2) and torch.equal(sy.view(torch.int32), s2.view(torch.int32))
    del y, qy, sy, q2, s2
    free()


def test_dgrad_output_past_2gib():
    """dX [33024][32768] bf16 = 2.16 GB (contraction over 256 output features)."""
    m, n, k, cut = 33024, 256, 32768, 20480
    print(f"[large rows] dgrad {m}x{n}x{k}", flush=True)
    qdy, sdy = act(m, n, 4)
    qw, sw = weight(n, k, 5)
    dx = jet.gemm_dgrad(qdy, sdy, qw, sw)
    da = jet.gemm_dgrad(*rows_of(qdy, sdy, 0, cut), qw, sw)
    assert torch.equal(dx[:cut].view(torch.int16), da.view(torch.int16))
    del da
    db = jet.gemm_dgrad(*rows_of(qdy, sdy, cut, m), qw, sw)
    assert torch.equal(dx[cut:].view(torch.int16), db.view(torch.int16))
    del db
    rng = np.random.default_rng(6)
    rows = np.sort(rng.choice(m, 8, replace=False))
    cols = np.sort(rng.choice(k, 64, replace=False))
    ref = oracle.gemm_dgrad_ref_at(host(qdy), host(sdy), host(qw), host(sw), rows, cols)
    check(host(dx[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)]), ref, "dgrad past 2 GiB")
    del dx
    free()


@pytest.mark.parametrize("f32", [False, True])
def test_wgrad_row_operand_past_2gib(f32):
    """dY^T [32768][65792] codes = 2.16 GB over 65792 tokens: the output features
    run as row ranges; the reference splits them at 12288.  fp32 output: written,
    then accumulated onto."""
    n, m, k, cut = 32768, 65792, 256, 12288
    print(f"[large rows] wgrad f32={f32} {n}x{m}x{k}", flush=True)
    qdyt, sdyt = act(n, m, 7)   # rows: output features; groups of 128 tokens
    qxt, sxt = act(k, m, 8)
    if f32:
        dw = torch.full((n, k), 0.25, dtype=torch.float32, device=DEV)
        jet.gemm_wgrad_f32(qdyt, sdyt, qxt, sxt, dw, accumulate=True)
        parts = []
        for r0, r1 in ((0, cut), (cut, n)):
            p = torch.full((r1 - r0, k), 0.25, dtype=torch.float32, device=DEV)
            jet.gemm_wgrad_f32(*rows_of(qdyt, sdyt, r0, r1), qxt, sxt, p, accumulate=True)
            parts.append(p)
        assert torch.equal(dw.view(torch.int32), torch.cat(parts).view(torch.int32))
    else:
        dw = jet.gemm_wgrad(qdyt, sdyt, qxt, sxt)
        parts = [jet.gemm_wgrad(*rows_of(qdyt, sdyt, r0, r1), qxt, sxt) for r0, r1 in ((0, cut), (cut, n))]
        assert torch.equal(dw.view(torch.int16), torch.cat(parts).view(torch.int16))
        rng = np.random.default_rng(9)
        rows = np.sort(rng.choice(n, 6, replace=False))
        cols = np.sort(rng.choice(k, 48, replace=False))
        qr, sr = host(qdyt[torch.from_numpy(rows).to(DEV)]), host(sdyt[:, torch.from_numpy(rows).to(DEV)])
        ref = oracle.gemm_wgrad_ref_at(qr, sr, host(qxt), host(sxt), np.arange(len(rows)), cols)
        check(host(dw[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)]), ref,
              "wgrad past 2 GiB")
    del dw, parts, qdyt, sdyt
    free()


def test_fprop_swiglu_quant_output_past_2gib():
    """The fused gate+up FProp + SwiGLU + quantisation with codes qh [131328][16384]
    = 2.15 GB: codes and scales equal to two separate calls on a different row
    split."""
    m, n, k, cut = 131328, 32768, 256, 50000
    print(f"[large rows] fprop_swiglu_quant {m}x{n}x{k}", flush=True)
    qx, sx = act(m, k, 10)
    qw, sw = weight(n, k, 11)
    qh, sh = jet.gemm_fprop_swiglu_quant(qx, sx, qw, sw)
    qa, sa = jet.gemm_fprop_swiglu_quant(*rows_of(qx, sx, 0, cut), qw, sw)
    assert torch.equal(qh[:cut], qa) and torch.equal(sh[:, :cut].view(torch.int32), sa.view(torch.int32))
    del qa, sa
    qb, sb = jet.gemm_fprop_swiglu_quant(*rows_of(qx, sx, cut, m), qw, sw)
    assert torch.equal(qh[cut:], qb) and torch.equal(sh[:, cut:].view(torch.int32), sb.view(torch.int32))
    del qb, sb, qh, sh
    free()
