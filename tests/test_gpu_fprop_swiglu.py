"""GPU parity of gemm_fprop_swiglu_quant: the gate+up FProp whose epilogue
applies SwiGLU and the 1x128 quantisation (no bf16 gate+up output written).

It must equal swiglu_quant(gemm_fprop(...)) bit for bit, and the oracle's
swiglu_quant of gemm_fprop's bf16 output bit for bit, with that bf16 output
within the GEMM tolerance of the oracle's fp64 product.  Shapes cover one tile,
ragged rows, odd K-block counts (one tile per workgroup) and even ones (one
workgroup per CU looping over tiles), the Qwen3-8B, Llama-3.1-8B and Qwen3-32B
gate+up widths.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Guarded, f32_dev, host, u8_dev
import quantized_rl_amd as jet

pytestmark = pytest.mark.gpu


def operands(m, n, k, seed):
    rng = np.random.default_rng(seed)
    qx = oracle.e4m3_encode((rng.standard_normal((m, k)) * 100).astype(np.float32))
    qw = oracle.e4m3_encode((rng.standard_normal((n, k)) * 100).astype(np.float32))
    sx = (rng.uniform(0.5, 2.0, (k // 128, m)) * 2.0 ** -9).astype(np.float32)
    sw = (rng.uniform(0.5, 2.0, (n // 128, k // 128)) * 2.0 ** -7).astype(np.float32)
    return qx, sx, qw, sw


def run_both(m, n, k, seed):
    print(f"[fprop_swiglu] M={m} N={n} K={k}", flush=True)
    qx, sx, qw, sw = operands(m, n, k, seed)
    d = [u8_dev(qx), f32_dev(sx), u8_dev(qw), f32_dev(sw)]
    qh, sh = jet.gemm_fprop_swiglu_quant(*d)
    y = jet.gemm_fprop(*d)
    q2, s2 = jet.swiglu_quant(y)
    torch.cuda.synchronize()
    return host(qh), host(sh), host(q2), host(s2), host(y), (qx, sx, qw, sw)


@pytest.mark.parametrize("m,n,k", [(256, 256, 128), (300, 512, 384), (1000, 768, 256), (64, 1024, 512),
                                   (2048, 4096, 1024)])
def test_matches_swiglu_of_fprop_and_the_oracle(m, n, k):
    qh, sh, q2, s2, y, (qx, sx, qw, sw) = run_both(m, n, k, m + n + k)
    assert np.array_equal(qh, q2) and np.array_equal(sh.view(np.uint32), s2.view(np.uint32))
    qo, so = oracle.swiglu_quant(y)
    assert np.array_equal(qh, qo) and np.array_equal(sh.view(np.uint32), so.view(np.uint32))
    r = oracle.check_gemm(y, oracle.gemm_fprop_ref(qx, sx, qw, sw))
    assert r["ok"], r


@pytest.mark.parametrize("m,i,k", [(8192, 12288, 4096), (16384, 14336, 4096), (8192, 12800, 5120)])
def test_model_shapes_match_swiglu_of_fprop(m, i, k):
    """Qwen3-8B, Llama-3.1-8B and Qwen3-32B (half) gate+up at training batch sizes,
    against the two-kernel path on the GPU, and the oracle on sampled rows."""
    qh, sh, q2, s2, y, _ = run_both(m, 2 * i, k, 7)
    assert np.array_equal(qh, q2) and np.array_equal(sh.view(np.uint32), s2.view(np.uint32))
    rows = np.sort(np.random.default_rng(i).choice(m, 16, replace=False))
    qo, so = oracle.swiglu_quant(y[rows])
    assert np.array_equal(qh[rows], qo) and np.array_equal(sh[:, rows].view(np.uint32), so.view(np.uint32))


def test_guards_empty_contraction_and_no_rows():
    m, n, k = 200, 512, 256
    qx, sx, qw, sw = operands(m, n, k, 3)
    qg, sg = Guarded((m, n // 2), torch.uint8), Guarded((n // 256, m), torch.float32)
    jet.gemm_fprop_swiglu_quant(u8_dev(qx), f32_dev(sx), u8_dev(qw), f32_dev(sw), qg.t, sg.t)
    torch.cuda.synchronize()
    assert qg.intact() and sg.intact()
    # K = 0: the product is zero, so is h: codes 0, scales 1
    e8, ef = torch.empty((m, 0), dtype=torch.uint8, device="cuda:0"), torch.empty((0, m), dtype=torch.float32,
                                                                                  device="cuda:0")
    w8, wf = torch.empty((n, 0), dtype=torch.uint8, device="cuda:0"), torch.empty((n // 128, 0), dtype=torch.float32,
                                                                                  device="cuda:0")
    q0, s0 = jet.gemm_fprop_swiglu_quant(e8, ef, w8, wf)
    assert np.all(host(q0) == 0) and np.all(host(s0) == 1.0)
    qm, smm = jet.gemm_fprop_swiglu_quant(torch.empty((0, k), dtype=torch.uint8, device="cuda:0"),
                                          torch.empty((k // 128, 0), dtype=torch.float32, device="cuda:0"),
                                          u8_dev(qw), f32_dev(sw))
    assert qm.shape == (0, n // 2)
