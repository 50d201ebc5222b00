"""Host checks of the device helpers that must round exactly (no GPU).

The quantisation kernels compute fl32(x / S) as fl32(fl64(x * inv)), with inv
within one fp64 ulp of 1/S from two Newton-Raphson steps on v_rcp_f64's seed
(recip_nr; the host drives it with seeds perturbed by +-2^-14), S = fl32(amax /
448) as fl32(fl64(amax * fl64(1/448))), the RMSNorm factor 1 / sqrt as the fp32
rounding of the same refined reciprocal, and the square root with an exact
midpoint test; all are compiled here for the host from the same header and
compared bit for bit with x86's IEEE fp32 (and fp64) division and square root.
"""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_exact_math_helpers(tmp_path):
    exe = tmp_path / "exact_math_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "exact_math_check.cpp")], check=True)
    res = subprocess.run([str(exe), "5"], capture_output=True, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    for line in res.stdout.splitlines():
        assert line.endswith(" 0 mismatches"), line
