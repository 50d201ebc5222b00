"""Exhaustive GPU check of the two conversions the kernels take from the
hardware: the E4M3 cast (v_med3 clamp + v_cvt_pk_fp8_f32, as every quantiser
writes its codes) and the packed bf16 rounding of the GEMM epilogues
(v_cvt_pk_bf16_f32), on all 2^32 fp32 bit patterns except NaNs, against the
integer definitions of tests/gpu_probe/cast_ref.hpp (themselves tied to the
oracle's E4M3 encoder and to torch's bf16 rounding by tests/test_cast_ref.py)."""

import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "gpu_probe", "libcast_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location("build_probe", os.path.join(HERE, "gpu_probe", "build_probe.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    lib = ctypes.CDLL(LIB)
    for fn in (lib.probe_e4m3_all_fp32, lib.probe_bf16_all_fp32):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("which", ["e4m3", "bf16"])
def test_conversion_on_every_fp32_pattern(probe, which):
    bad = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    first = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    fn = probe.probe_e4m3_all_fp32 if which == "e4m3" else probe.probe_bf16_all_fp32
    stream = torch.cuda.current_stream().cuda_stream
    assert fn(bad.data_ptr(), first.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    n, f = int(bad.item()), int(first.item()) & 0xFFFFFFFF
    assert n == 0, f"{which}: {n} mismatches, first at fp32 bits {f:#010x}"
