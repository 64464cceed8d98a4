"""Host checks of the device math the kernels share (no GPU needed).

The final draw's weights use the fp64 exponential exp2_neg (2^f = 1 + f q(f)
on |f| <= 1/2 with q the degree-8 Chebyshev interpolant of (2^f - 1) / f,
scaled by 2^n); its error bound is pinned here against long-double exp2l,
compiled from the same header the kernels include."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "rejection_sampling_verify_15_amd", "csrc")


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc is needed to build the host check")
def test_exp2_error_bound(tmp_path):
    exe = tmp_path / "exp2_check"
    cmd = [_hipcc(), "-O2", "-std=c++17", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           "-o", str(exe), os.path.join(HERE, "exp2_check.cpp")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    vals = dict(zip(out[0::2], out[1::2]))
    assert vals["zero_ok"] == "1"
    assert int(vals["count"]) > 5_000_000
    # Chebyshev interpolation of (2^f - 1) / f at nine nodes on [-1/2, 1/2]:
    # the polynomial itself (in exact arithmetic) is off by 3.70e-14 relative
    # at f = -1/2, its worst point; rounding the coefficients and the Horner
    # steps add a few ulps.  The inverse-CDF draw needs about 1e-10.
    assert float(vals["max_rel"]) < 3.8e-14, vals
