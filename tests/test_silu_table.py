"""The SiLU table that the kernels compile in (generated at build time by
quantized_rl_amd/csrc/silu_table_gen.cpp with the C library's exp; used by
swiglu_quant and the fused gate+up FProp epilogue) equals the oracle's silu, bit
for bit, on every one of its 8192 arguments; the closed forms outside its range
are checked on the GPU against the oracle on every finite bf16 value."""

import os
import subprocess

import numpy as np

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "quantized_rl_amd", "csrc", "silu_table_gen.cpp")


def test_generated_silu_table_matches_the_oracle(tmp_path):
    exe, out = tmp_path / "gen", tmp_path / "silu_table.inc"
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-o", str(exe), GEN], check=True)
    subprocess.run([str(exe), str(out)], check=True)
    tab = np.array([int(ln.strip().rstrip(",").rstrip("u"), 16) for ln in open(out) if ln.startswith("0x")],
                   np.uint32)
    assert tab.size == 8192
    i = np.arange(8192, dtype=np.uint32)
    bits = (((i >> 12) << 15) | ((((i >> 7) & 31) + 102) << 7) | (i & 127)) << 16
    g = bits.view(np.float32)
    assert np.all((np.abs(g) >= 2.0 ** -25) & (np.abs(g) < 128))
    assert np.array_equal(tab, oracle.silu_f32(g).view(np.uint32))
