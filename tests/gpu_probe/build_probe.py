"""Build the GPU conversion probe (test infrastructure) in-tree with hipcc:
tests/gpu_probe/libcast_probe.so, loaded only by tests/test_gpu_casts.py."""

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libcast_probe.so")

# the library's own code-generation flags (quantized_rl_amd/build.py), so the
# conversions are compiled as they are in its kernels
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB + ".tmp"
    res = subprocess.run([exe, *FLAGS, "-x", "hip", os.path.join(HERE, "cast_probe.hip"), "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on the conversion probe:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
