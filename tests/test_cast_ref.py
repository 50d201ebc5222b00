"""The integer conversion definitions the GPU probe holds the hardware to
(tests/gpu_probe/cast_ref.hpp), tied on the CPU to the oracle's E4M3 encoder
(nearest value in the OCP E4M3FN table, ties to the even code, saturating;
paper.rainbus.top, section "FP8 量化 (E4M3 格式)") and to torch's fp32 -> bf16
rounding (library), on every E4M3 value and rounding midpoint +-8 fp32 ulps,
the whole subnormal-E4M3 range in steps of 2^-20, and a million random fp32
patterns."""

import os
import subprocess

import numpy as np
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE = os.path.join(HERE, "gpu_probe")


def patterns():
    tab = np.array([float(oracle.e4m3_decode(np.array([c], np.uint8))[0]) for c in range(0x7F)])
    mids = (tab[:-1] + tab[1:]) / 2
    pts = np.concatenate([tab, mids, [448.0, 464.0, 480.0, 1e30, 3.4e38, 2.0 ** -149, 2.0 ** -126]])
    base = pts.astype(np.float32).view(np.uint32).astype(np.int64)
    near = (base[:, None] + np.arange(-8, 9)[None, :]).ravel()
    near = near[(near >= 0) & (near <= 0x7F800000)].astype(np.uint32)
    sub = (np.arange(0, 2 ** 11) * np.float32(2.0 ** -20)).astype(np.float32).view(np.uint32)
    rnd = np.random.default_rng(8).integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([near, sub, rnd])
    u = np.concatenate([u, u ^ np.uint32(0x80000000)])
    return u[(u & np.uint32(0x7FFFFFFF)) < np.uint32(0x7F800000)]  # finite (the oracle takes no inf)


def test_cast_ref_matches_oracle_and_torch(tmp_path):
    exe = tmp_path / "cast_ref_dump"
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", str(exe), os.path.join(PROBE, "cast_ref_dump.cpp")],
                   check=True)
    u = patterns()
    out = subprocess.run([str(exe)], input=u.astype("<u4").tobytes(), capture_output=True, check=True).stdout
    codes = np.frombuffer(out[:u.size], np.uint8)
    bf = np.frombuffer(out[u.size:], "<u2")
    x = u.view(np.float32)
    want = oracle.e4m3_encode(x)
    bad = np.nonzero(codes != want)[0]
    assert bad.size == 0, [(hex(int(u[i])), hex(int(codes[i])), hex(int(want[i]))) for i in bad[:5]]
    tb = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, tb)
