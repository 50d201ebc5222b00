"""Build the gfx950 FP8 linear-layer library (libjetfp8.so) in-tree with hipcc.

Usage: ``python -m quantized_rl_amd.build`` (or ``build()`` from Python).
The library lands next to this file; it is always rebuilt when called.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libjetfp8.so")
SOURCES = ["api.cpp", "quant_kernels.hip", "gemm_kernels.hip", "norm_kernels.hip", "swiglu_kernels.hip"]

# -ffp-contract=off: every fp32 multiply and add of the quantisers is its own
#   rounding step (no fused multiply-add), as their definitions state.
# -fhip-fp32-correctly-rounded-divide-sqrt: IEEE division and square root.
# -packed-fp32-ops disabled: no v_pk_{add,mul,fma}_f32 in generated code.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the decode and 128 x 128 kernels rescale
    # every block product with VALU FMAs, which otherwise first copy it out of
    # the accumulation registers (v_accvgpr_read, 4 per MFMA)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the library needs ROCm's hipcc to build")
    return exe


def gen_silu_table():
    """Run the build-time generator of the SiLU table (host C++) into csrc/silu_table.inc."""
    exe = os.path.join(CSRC, "silu_table_gen")
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        raise RuntimeError("a host C++ compiler (g++) is needed to generate the SiLU table")
    subprocess.run([cxx, "-O2", "-std=c++17", "-ffp-contract=off", "-o", exe,
                    os.path.join(CSRC, "silu_table_gen.cpp")], check=True)
    out = os.path.join(CSRC, "silu_table.inc")
    subprocess.run([exe, out + ".tmp"], check=True)
    os.replace(out + ".tmp", out)
    os.remove(exe)
    return out


def build(verbose=False):
    gen_silu_table()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-x", "hip", *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(
        ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln
    )
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    print(LIB)
