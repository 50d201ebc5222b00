"""The C ABI from plain C: include/jetfp8.h compiles as C11, a C program links
against libjetfp8.so and the HIP runtime (CPU), and on the GPU that program's
outputs match the oracle (quantisers bit for bit, FProp to the GEMM tolerance)."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from quantized_rl_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "c_abi_check.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_program(out):
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", libdir, "-ljetfp8", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{libdir}:{os.path.join(ROCM, 'lib')}", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_header_is_plain_c():
    r = subprocess.run(["gcc", "-fsyntax-only", "-std=c11", "-Wall", "-Wextra", "-Werror", "-x", "c",
                        os.path.join(ROOT, "include", "jetfp8.h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_links(jetlib, tmp_path):
    build_c_program(str(tmp_path / "c_abi_check"))


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["linear_small", "rollout_64"])
def test_c_program_matches_the_oracle(jetlib, tmp_path, case):
    """linear_small: X [256, 512] with outlier channels, W [384, 512] (gemm_fprop_splitk
    needs no workspace there); rollout_64: X [64, 1024], W [384, 1024], where it splits
    K in two through the workspace the program allocates."""
    if case == "linear_small":
        d = synth.linear_small()
        x, w = d["x"], d["w"]
    else:
        x = synth.random_bf16((64, 1024), seed=64)
        w = synth.random_bf16((384, 1024), seed=65, std=0.02)
    (m, k), n = x.shape, w.shape[0]
    exe = str(tmp_path / "c_abi_check")
    build_c_program(exe)
    x.astype(np.uint16).tofile(tmp_path / "x.bin")
    w.astype(np.uint16).tofile(tmp_path / "w.bin")
    prefix = str(tmp_path) + os.sep
    r = subprocess.run([exe, str(m), str(k), str(n), str(tmp_path / "x.bin"), str(tmp_path / "w.bin"), prefix],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    q = np.fromfile(tmp_path / "qx.bin", dtype=np.uint8).reshape(m, k)
    s = np.fromfile(tmp_path / "sx.bin", dtype=np.float32).reshape(k // 128, m)
    y = np.fromfile(tmp_path / "y.bin", dtype=np.uint16).reshape(m, n)
    qo, so = oracle.quant_act_1x128(x)
    assert np.array_equal(q, qo) and np.array_equal(s.view(np.uint32), so.view(np.uint32))
    qwo, swo = oracle.quant_weight_128x128(w)
    ref = oracle.gemm_fprop_ref(qo, so, qwo, swo)
    res = oracle.check_gemm(y, ref)
    assert res["ok"], res
    y2 = np.fromfile(tmp_path / "y_splitk.bin", dtype=np.uint16).reshape(m, n)
    res = oracle.check_gemm(y2, ref)
    assert res["ok"], res
