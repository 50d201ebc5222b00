"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and its host-side validation rejects bad arguments before enqueuing anything.

Pointers here are fake integers; every call either fails validation or has an
empty output, so no kernel is ever launched -- except the two checks that
adjacent buffers pass validation, which run only where no GPU is visible (the
launch then fails with ELAUNCH instead of touching memory).
"""

import os
import re
import subprocess

import pytest

from quantized_rl_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "jetfp8.h")
OK, EINVAL, EALIGN, ENULL, EALIAS = 0, 1, 2, 3, 4
A = 1 << 20  # fake, 16-byte aligned addresses, far apart
P = [A * (i + 1) for i in range(10)]


def no_gpu():
    import torch
    return torch.cuda.device_count() == 0


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:int|int64_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_seven_entry_points():
    names = declared_functions()
    for n in ["quantize_act_1x128", "quantize_weight_128x128", "rmsnorm_quant",
              "requant_transpose_128x1", "gemm_fprop", "gemm_dgrad", "gemm_wgrad", "gemm_wgrad_f32",
              "rmsnorm_quant_rstd", "rmsnorm_backward", "rmsnorm_backward_workspace_bytes",
              "jetfp8_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol(jetlib):
    for name in declared_functions():
        assert hasattr(jetlib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported


def test_status_strings(jetlib):
    for code in range(7):
        assert jetlib.jetfp8_status_string(code)
    assert jetlib.jetfp8_status_string(99) == b"unknown status"


def c(name, *args):
    return _lib.call_raw(name, *args)


def test_quantize_act_validation(jetlib):
    assert c("quantize_act_1x128", P[0], 4, 100, P[1], P[2], 0) == EINVAL
    assert c("quantize_act_1x128", P[0], -1, 128, P[1], P[2], 0) == EINVAL
    assert c("quantize_act_1x128", P[0], 1 << 31, 128, P[1], P[2], 0) == EINVAL
    assert c("quantize_act_1x128", 0, 4, 128, P[1], P[2], 0) == ENULL
    assert c("quantize_act_1x128", P[0], 4, 128, 0, P[2], 0) == ENULL
    assert c("quantize_act_1x128", P[0] + 8, 4, 128, P[1], P[2], 0) == EALIGN
    assert c("quantize_act_1x128", P[0], 4, 128, P[0] + 512, P[2], 0) == EALIAS  # q inside x
    assert c("quantize_act_1x128", P[0], 4, 128, P[1], P[1] + 256, 0) == EALIAS  # s inside q
    if no_gpu():
        assert c("quantize_act_1x128", P[0], 4, 128, P[0] + 1024, P[2], 0) != EALIAS  # adjacent is fine
    assert c("quantize_act_1x128", 0, 0, 128, 0, 0, 0) == OK  # empty: nothing to do


def test_quantize_weight_and_rmsnorm_validation(jetlib):
    assert c("quantize_weight_128x128", P[0], 100, 128, P[1], P[2], 0) == EINVAL
    assert c("quantize_weight_128x128", P[0], 128, 100, P[1], P[2], 0) == EINVAL
    assert c("quantize_weight_128x128", P[0], 128, 128, P[1], P[1] + 16384 - 16, 0) == EALIAS
    assert c("rmsnorm_quant", P[0], P[1], 4, 0, 1e-6, P[2], P[3], 0) == EINVAL
    assert c("rmsnorm_quant", P[0], P[1], 4, 65536 + 128, 1e-6, P[2], P[3], 0) == EINVAL
    assert c("rmsnorm_quant", P[0], 0, 4, 128, 1e-6, P[2], P[3], 0) == ENULL
    assert c("rmsnorm_quant", P[0], P[1], 4, 128, 1e-6, P[1], P[3], 0) == EALIAS  # q over gamma
    assert c("rmsnorm_quant", 0, P[1], 0, 128, 1e-6, 0, 0, 0) == OK


def test_requant_validation(jetlib):
    assert c("requant_transpose_128x1", P[0], P[1], 200, 128, P[2], P[3], 0) == EINVAL
    assert c("requant_transpose_128x1", P[0], P[1], 128, 200, P[2], P[3], 0) == EINVAL
    assert c("requant_transpose_128x1", P[0], P[1], 128, 128, P[2], P[2] + 64, 0) == EALIAS
    assert c("requant_transpose_128x1", P[0], P[1] + 4, 128, 128, P[2], P[3], 0) == EALIGN
    assert c("requant_transpose_128x1", 0, 0, 0, 128, 0, 0, 0) == OK


def test_gemm_size_limit(jetlib):
    """Row operands and outputs of any size run as row ranges (tested on the GPU);
    what stays unsupported is a column operand of 2^31 bytes or more, or 512 rows
    of the row operand or of the output reaching 2^31 bytes."""
    EUNSUP = 5
    Q = [(i + 1) << 40 for i in range(8)]  # fake addresses far enough apart for 4 GiB tensors
    # the weight [N][K] at 2^31 bytes
    assert c("gemm_fprop", Q[0], Q[1], Q[2], Q[3], 16, 1 << 16, 1 << 15, Q[4], 0) == EUNSUP
    assert c("gemm_dgrad", Q[0], Q[1], Q[2], Q[3], 16, 1 << 16, 1 << 15, Q[4], 0) == EUNSUP
    assert c("gemm_fprop_quant", Q[0], Q[1], Q[2], Q[3], 16, 1 << 16, 1 << 15, Q[4], Q[5], Q[6], 0) == EUNSUP
    assert c("gemm_fprop_swiglu_quant", Q[0], Q[1], Q[2], Q[3], 16, 1 << 16, 1 << 15, Q[4], Q[5], 0) == EUNSUP
    # WGrad's column operand X^T [K][M]: 2^20 tokens x 4096 features = 4 GiB
    assert c("gemm_wgrad", Q[0], Q[1], Q[2], Q[3], 1 << 20, 128, 4096, Q[4], 0) == EUNSUP
    assert c("gemm_wgrad_f32", Q[0], Q[1], Q[2], Q[3], 1 << 20, 128, 4096, Q[4], 0, 0) == EUNSUP
    # 512 output rows of 2^21 bf16 columns reach 2^31 bytes (the weight itself fits)
    assert c("gemm_fprop", Q[0], Q[1], Q[2], Q[3], 16, 1 << 21, 128, Q[4], 0) == EUNSUP
    # a 2^22-byte contraction: 512 rows of the row operand reach 2^31 bytes
    assert c("gemm_dgrad", Q[0], Q[1], Q[2], Q[3], 16, 1 << 22, 128, Q[4], 0) == EUNSUP


def test_gemm_fprop_quant_validation(jetlib):
    f = "gemm_fprop_quant"
    assert c(f, P[0], P[1], P[2], P[3], 16, 100, 128, P[4], P[5], P[6], 0) == EINVAL
    assert c(f, P[0], P[1], P[2], P[3], 16, 128, 128, P[4], 0, P[6], 0) == ENULL     # qy missing
    assert c(f, P[0], P[1], P[2], P[3], 16, 128, 128, P[4], P[4], P[6], 0) == EALIAS  # qy overlaps y
    assert c(f, P[0], P[1], P[2], P[3], 16, 128, 128, P[4], P[5], P[0], 0) == EALIAS  # sy overlaps qx
    assert c(f, P[0], P[1], P[2], P[3], 16, 128, 128, P[4], P[5], P[6] + 8, 0) == EALIGN
    assert c(f, 0, 0, P[2], P[3], 0, 128, 128, 0, 0, 0, 0) == OK  # M = 0: nothing to do


def test_gemm_validation(jetlib):
    # fprop(qx, sx, qw, sw, M, N, K, y)
    assert c("gemm_fprop", P[0], P[1], P[2], P[3], 16, 100, 128, P[4], 0) == EINVAL
    assert c("gemm_fprop", P[0], P[1], P[2], P[3], 16, 128, 64, P[4], 0) == EINVAL
    assert c("gemm_fprop", P[0], P[1], P[2], P[3], 16, 128, 128, P[0], 0) == EALIAS
    assert c("gemm_fprop", P[0], P[1], 0, P[3], 16, 128, 128, P[4], 0) == ENULL
    assert c("gemm_fprop", P[0], P[1], P[2], P[3] + 4, 16, 128, 128, P[4], 0) == EALIGN
    assert c("gemm_fprop", 0, 0, P[2], P[3], 0, 128, 128, 0, 0) == OK  # M = 0
    assert c("gemm_dgrad", P[0], P[1], P[2], P[3], 16, 128, 96, P[4], 0) == EINVAL
    assert c("gemm_dgrad", P[0], P[1], P[2], P[3], 16, 128, 128, P[2] + 32, 0) == EALIAS
    assert c("gemm_dgrad", 0, 0, P[2], P[3], 0, 128, 128, 0, 0) == OK
    # wgrad(qdyt, sdyt, qxt, sxt, M, N, K, dw): M must be a multiple of 128
    assert c("gemm_wgrad", P[0], P[1], P[2], P[3], 100, 128, 128, P[4], 0) == EINVAL
    assert c("gemm_wgrad", P[0], P[1], P[2], P[3], 128, 128, 128, P[3], 0) == EALIAS
    assert c("gemm_wgrad", P[0], P[1], P[2], P[3], 128, 0, 128, 0, 0) == OK  # N = 0: empty output


def test_gemm_wgrad_f32_validation(jetlib):
    f = "gemm_wgrad_f32"
    # wgrad_f32(qdyt, sdyt, qxt, sxt, M, N, K, dw, accumulate)
    assert c(f, P[0], P[1], P[2], P[3], 100, 128, 128, P[4], 0, 0) == EINVAL   # M % 128
    assert c(f, P[0], P[1], P[2], P[3], 128, 128, 128, P[4], 2, 0) == EINVAL   # accumulate not 0/1
    assert c(f, P[0], P[1], P[2], P[3], 128, 128, 128, P[4], -1, 0) == EINVAL
    assert c(f, P[0], P[1], P[2], P[3], 128, 128, 128, 0, 0, 0) == ENULL
    assert c(f, P[0], P[1], P[2], P[3], 128, 128, 128, P[4] + 8, 1, 0) == EALIGN
    assert c(f, P[0], P[1], P[2], P[3], 128, 128, 128, P[3] - 16, 0, 0) == EALIAS  # dw runs into sxt
    assert c(f, P[0], P[1], P[2], P[3], 128, 0, 128, 0, 1, 0) == OK  # N = 0: empty output
    # 4-byte output elements: 512 rows of dW [128, 2^20] fp32 reach 2^31 bytes (in bf16 they would not)
    Q = [(i + 1) << 40 for i in range(8)]
    assert c(f, Q[0], Q[1], Q[2], Q[3], 128, 128, 1 << 20, Q[4], 0, 0) == 5


def test_rmsnorm_rstd_and_backward_validation(jetlib):
    f = "rmsnorm_quant_rstd"
    assert c(f, P[0], P[1], 4, 100, 1e-6, P[2], P[3], P[4], 0) == EINVAL
    assert c(f, P[0], P[1], 4, 128, 1e-6, P[2], P[3], 0, 0) == ENULL          # rstd missing
    assert c(f, P[0], P[1], 16, 128, 1e-6, P[2], P[3], P[3] + 16, 0) == EALIAS  # rstd overlaps s
    assert c(f, 0, P[1], 0, 128, 1e-6, 0, 0, 0, 0) == OK
    ws = _lib.rmsnorm_backward_workspace_bytes
    # one row of K floats per workgroup of R rows, R = 2 ceil(M / 512) in 1..32
    assert ws(8192, 4096) == 4 * 256 * 4096 and ws(1, 128) == 4 * 128 and ws(0, 128) == 0
    assert ws(256, 4096) == 4 * 128 * 4096 and ws(2000, 128) == 4 * 250 * 128 and ws(65536, 128) == 4 * 2048 * 128
    assert ws(4, 100) == -1 and ws(4, 24576 + 128) == -1 and ws(-1, 128) == -1 and ws(4, 24576) > 0
    b = "rmsnorm_backward"
    # (x, gamma, rstd, dy, M, K, dx, dgamma, workspace)
    assert c(b, P[0], P[1], P[2], P[3], 4, 24704, P[4], P[5], P[6], 0) == EINVAL  # K > 24576
    assert c(b, P[0], P[1], P[2], P[3], 4, 128, P[4], P[5], 0, 0) == ENULL      # workspace missing
    assert c(b, P[0], P[1], P[2], P[3], 4, 128, P[4], P[5], P[4] + 512, 0) == EALIAS  # workspace over dx
    assert c(b, P[0], P[1], P[2], P[3], 4, 128, P[3], P[5], P[6], 0) == EALIAS  # dx over dy
    assert c(b, P[0], P[1], P[2], P[3], 4, 128, P[4], P[5] + 4, P[6], 0) == EALIGN


def test_gemm_fprop_splitk_validation(jetlib):
    ws = _lib.gemm_fprop_splitk_workspace_bytes
    # S * M * N * 4 bytes: S shares of K (dividing K/128, >= 4 blocks each, at most 512
    # workgroups) when there are fewer 128 x 128 tiles than 256 and 33 <= M <= 256, or
    # 17 <= M <= 32 with K >= 8192
    assert ws(256, 6144, 4096) == 4 * 256 * 6144 * 4      # 8B QKV: 96 tiles, 32 blocks
    assert ws(256, 4096, 12288) == 8 * 256 * 4096 * 4     # 8B down: 64 tiles, 96 blocks
    assert ws(128, 6144, 4096) == 8 * 128 * 6144 * 4      # 48 tiles
    assert ws(256, 5120, 12800) == 5 * 256 * 5120 * 4     # 32B down: 80 tiles, 100 blocks
    assert ws(256, 24576, 4096) == 0                       # 384 tiles fill the chip
    assert ws(64, 6144, 4096) == 8 * 64 * 6144 * 4       # 48 tiles
    assert ws(32, 4096, 12288) == 16 * 32 * 4096 * 4     # long K at 17..32 rows
    assert ws(16, 6144, 4096) == ws(16, 4096, 12288) == ws(32, 6144, 4096) == 0
    assert ws(257, 6144, 4096) == ws(200, 384, 512) == 0
    raw = jetlib.gemm_fprop_splitk_workspace_bytes
    assert raw(16, 100, 128) == -1 and raw(-1, 128, 128) == -1 and raw(16, 128, 64) == -1
    with pytest.raises(_lib.JetFP8Error):
        ws(16, 100, 128)
    f = "gemm_fprop_splitk"
    need = ws(256, 6144, 4096)
    # (qx, sx, qw, sw, M, N, K, y, workspace, workspace_bytes)
    assert c(f, P[0], P[1], P[2], P[3], 256, 6144, 4096, P[4], P[5], need - 4, 0) == EINVAL  # too small
    assert c(f, P[0], P[1], P[2], P[3], 256, 6144, 4096, P[4], 0, need, 0) == ENULL
    assert c(f, P[0], P[1], P[2], P[3], 256, 6144, 4096, P[4], P[5] + 8, need, 0) == EALIGN
    Q = [(i + 1) << 36 for i in range(8)]
    assert c(f, Q[0], Q[1], Q[2], Q[3], 256, 6144, 4096, Q[4], Q[4] + 1024, need, 0) == EALIAS  # over y
    assert c(f, Q[0], Q[1], Q[2], Q[3], 256, 6144, 4096, Q[4], Q[2], need, 0) == EALIAS         # over qw
    assert c(f, P[0], P[1], P[2], P[3], 16, 100, 128, P[4], P[5], 0, 0) == EINVAL
    assert c(f, 0, 0, P[2], P[3], 0, 128, 128, 0, 0, 0, 0) == OK  # M = 0: nothing to do


def test_swiglu_quant_validation(jetlib):
    # (y [M][2I], M, I, q [M][I], s [I/128][M])
    assert "swiglu_quant" in declared_functions()
    assert c("swiglu_quant", P[0], 4, 100, P[1], P[2], 0) == EINVAL        # I % 128
    assert c("swiglu_quant", P[0], -1, 128, P[1], P[2], 0) == EINVAL
    assert c("swiglu_quant", P[0], 4, 1 << 30, P[1], P[2], 0) == EINVAL    # 2I past 2^31 - 1
    assert c("swiglu_quant", 0, 4, 128, P[1], P[2], 0) == ENULL
    assert c("swiglu_quant", P[0], 4, 128, P[1] + 4, P[2], 0) == EALIGN
    assert c("swiglu_quant", P[0], 4, 128, P[0] + 1024, P[2], 0) == EALIAS  # q inside y (2 KB)
    if no_gpu():
        assert c("swiglu_quant", P[0], 4, 128, P[0] + 2048, P[2], 0) != EALIAS  # right after y
    assert c("swiglu_quant", P[0], 4, 128, P[1], P[1] + 256, 0) == EALIAS   # s inside q
    assert c("swiglu_quant", 0, 0, 128, 0, 0, 0) == OK


def test_fprop_splitk_noalloc_validation(jetlib):
    # (qx, sx, qw, sw, M, N, K, y)
    n = "gemm_fprop_splitk_noalloc"
    assert c(n, P[0], P[1], P[2], P[3], 256, 100, 4096, P[4], 0) == EINVAL      # N % 128
    assert c(n, P[0], P[1], P[2], P[3], 256, 4096, 4000, P[4], 0) == EINVAL     # K % 128
    assert c(n, P[0], P[1], P[2], P[3], 256, 4096, 4096, 0, 0) == ENULL          # no output
    assert c(n, P[0], P[1], P[2], P[3] + 8, 256, 4096, 4096, P[4], 0) == EALIGN
    assert c(n, P[0], P[1], P[2], P[3], 256, 4096, 4096, P[2] + 64, 0) == EALIAS  # y over qw
    assert c(n, 0, 0, P[2], P[3], 0, 4096, 4096, 0, 0) == OK                     # M = 0: nothing to do
    # the split rule never asks for more than the library's 32 MiB
    ws = _lib.gemm_fprop_splitk_workspace_bytes
    assert max(ws(m, nn, k) for m in (17, 33, 64, 100, 128, 200, 256) for nn in (4096, 6144, 8192, 16256)
               for k in (4096, 12288, 16384)) <= _lib.NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert "#define JETFP8_NOALLOC_SCRATCH_BYTES (32ll << 20)" in text


def test_fprop_swiglu_quant_validation(jetlib):
    # (qx, sx, qw, sw, M, N, K, qh, sh)
    n = "gemm_fprop_swiglu_quant"
    assert n in declared_functions()
    assert c(n, P[0], P[1], P[2], P[3], 256, 384, 256, P[4], P[5], 0) == EINVAL   # N % 256
    assert c(n, P[0], P[1], P[2], P[3], 256, 512, 200, P[4], P[5], 0) == EINVAL   # K % 128
    assert c(n, P[0], P[1], P[2], P[3], 256, 512, 256, 0, P[5], 0) == ENULL
    assert c(n, P[0], P[1], P[2], P[3], 256, 512, 256, P[4], P[5] + 4, 0) == EALIGN
    assert c(n, P[0], P[1], P[2], P[3], 256, 512, 256, P[4], P[4] + 1024, 0) == EALIAS  # sh inside qh
    B = [(i + 1) << 40 for i in range(6)]  # far apart: no overlap even for huge shapes
    assert c(n, B[0], B[1], B[2], B[3], 16, 1 << 16, 1 << 15, B[4], B[5], 0) == 5  # the weight at 2^31 bytes
    assert c(n, 0, 0, P[2], P[3], 0, 512, 256, 0, 0, 0) == OK


def test_pack_weight_rollout_and_fprop_packed_validation(jetlib):
    for n in ("pack_weight_rollout", "gemm_fprop_packed"):
        assert n in declared_functions()
    # (qw, N, K, qwp)
    p = "pack_weight_rollout"
    assert c(p, P[0], 100, 128, P[1], 0) == EINVAL                  # N % 128
    assert c(p, P[0], 128, 200, P[1], 0) == EINVAL                  # K % 128
    assert c(p, P[0], -128, 128, P[1], 0) == EINVAL
    assert c(p, 0, 128, 128, P[1], 0) == ENULL
    assert c(p, P[0], 128, 128, P[1] + 8, 0) == EALIGN
    assert c(p, P[0], 128, 128, P[0] + 8192, 0) == EALIAS            # qwp inside qw (16 KB)
    B = [(i + 1) << 40 for i in range(6)]
    assert c(p, B[0], 1 << 16, 1 << 15, B[1], 0) == 5               # 2^31 bytes: past 32-bit offsets
    assert c(p, 0, 0, 128, 0, 0) == OK and c(p, 0, 128, 0, 0, 0) == OK
    # (qx, sx, qwp, sw, M, N, K, y)
    f = "gemm_fprop_packed"
    assert c(f, P[0], P[1], P[2], P[3], 16, 100, 128, P[4], 0) == EINVAL       # N % 128
    assert c(f, P[0], P[1], P[2], P[3], 16, 128, 100, P[4], 0) == EINVAL       # K % 128
    assert c(f, P[0], P[1], P[2], P[3], 16, 128, 128, 0, 0) == ENULL
    assert c(f, P[0], P[1], P[2] + 4, P[3], 16, 128, 128, P[4], 0) == EALIGN
    assert c(f, P[0], P[1], P[2], P[3], 16, 128, 128, P[2] + 64, 0) == EALIAS  # y over qwp
    assert c(f, P[0], P[1], P[2], P[3], 257, 128, 128, P[4], 0) == 5           # more than 256 rows
    assert c(f, B[0], B[1], B[2], B[3], 16, 1 << 16, 1 << 15, B[4], 0) == 5    # weight past 2^31 bytes
    assert c(f, 0, 0, P[2], P[3], 0, 128, 128, 0, 0) == OK                      # M = 0: nothing to do
