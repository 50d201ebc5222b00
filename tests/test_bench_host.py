"""Host-side logic of bench.py: the roofline traffic record is used only for the
GEMM source it was measured on."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_record_parses_and_is_tied_to_the_source(tmp_path, monkeypatch):
    v = bench.measured_traffic("gemm_wgrad")
    assert v is None or (isinstance(v, int) and v > 0)
    assert bench.measured_traffic("no_such_kernel") is None
    rec = tmp_path / "rec.md"
    rec.write_text("    source_sha256 quantized_rl_amd/csrc/gemm_kernels.hip " + "0" * 64 + "\n"
                   "    traffic_bytes gemm_wgrad 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec))
    assert bench.measured_traffic("gemm_wgrad") is None  # hash differs: stale record
    import hashlib
    src = os.path.join(ROOT, "quantized_rl_amd", "csrc", "gemm_kernels.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    rec.write_text(f"    source_sha256 quantized_rl_amd/csrc/gemm_kernels.hip {h}\n"
                   "    traffic_bytes gemm_wgrad 123\n")
    assert bench.measured_traffic("gemm_wgrad") == 123
