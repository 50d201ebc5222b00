"""gemm_fprop_splitk_noalloc (split-K FProp through the library's own static
workspace, for callers that cannot allocate) against gemm_fprop_splitk with a
caller workspace: bit-identical outputs on two calls in a row, the second on a
smaller problem, and both within the GEMM tolerance of the oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import f32_dev, host, u8_dev
import quantized_rl_amd as jet

pytestmark = pytest.mark.gpu


def operands(m, n, k, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((m, k)).astype(np.float32) * np.float32(100)
    qx = oracle.e4m3_encode(v)
    qw = oracle.e4m3_encode(rng.standard_normal((n, k)).astype(np.float32) * np.float32(100))
    sx = (rng.uniform(0.5, 2.0, (k // 128, m)) * 2.0 ** -10).astype(np.float32)
    sw = (rng.uniform(0.5, 2.0, (n // 128, k // 128)) * 2.0 ** -8).astype(np.float32)
    return qx, sx, qw, sw


def run(m, n, k, seed):
    print(f"[no_alloc] M={m} N={n} K={k}", flush=True)
    qx, sx, qw, sw = operands(m, n, k, seed)
    d = [u8_dev(qx), f32_dev(sx), u8_dev(qw), f32_dev(sw)]
    need = jet.gemm_fprop_splitk_workspace_bytes(m, n, k)
    ws = torch.empty((max(need, 4) // 4,), dtype=torch.float32, device="cuda:0")
    y_ws = jet.gemm_fprop_splitk(*d, workspace=ws)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    jet.gemm_fprop_splitk_noalloc(*d, y)
    torch.cuda.synchronize()
    return host(y), host(y_ws), (qx, sx, qw, sw), need


def test_two_calls_in_a_row_second_smaller():
    y1, y1_ws, ops1, need1 = run(256, 4096, 12288, 1)   # the largest workspace: 32 MiB (S = 8)
    assert need1 == jet.NOALLOC_SCRATCH_BYTES
    y1_kept = y1.copy()
    y2, y2_ws, ops2, need2 = run(64, 6144, 4096, 2)     # 12 MiB (S = 8)
    assert 0 < need2 < need1
    assert np.array_equal(y1, y1_ws) and np.array_equal(y2, y2_ws)
    for y, (qx, sx, qw, sw), what in [(y1_kept, ops1, "first"), (y2, ops2, "second")]:
        r = oracle.check_gemm(y, oracle.gemm_fprop_ref(qx, sx, qw, sw))
        assert r["ok"], f"{what} call: {r}"


def test_unsplit_shape_runs_gemm_fprop():
    m, n, k = 16, 6144, 4096   # decode batch: no K split, no scratch
    assert jet.gemm_fprop_splitk_workspace_bytes(m, n, k) == 0
    y, y_ws, (qx, sx, qw, sw), _ = run(m, n, k, 3)
    assert np.array_equal(y, y_ws)
    y_plain = host(jet.gemm_fprop(u8_dev(qx), f32_dev(sx), u8_dev(qw), f32_dev(sw)))
    assert np.array_equal(y, y_plain)
