"""Host check of the bulk write's code cutoffs.

The bulk demotion kernel turns level_code(fl((v - zero) / scale)) into three
comparisons of v - zero with per-group float cutoffs (code_cuts / code_cut in
csrc/oscar_internal.h).  tests/host/code_cut_check.cpp compiles that same
header for the host and compares the cutoff form with the correctly rounded
quotient on millions of cases around every cutoff, at rounding ties, and over
uniform-grid, random-codebook and subnormal thresholds.  The codes themselves
are checked against the oracle by the GPU parity tests; this test covers the
rare boundary and tie cases that random data does not reach.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_cutoffs_equal_rounded_quotient(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "code_cut_check"
    src = os.path.join(ROOT, "tests", "host", "code_cut_check.cpp")
    subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "bit_rotated_kv_int2_amd", "csrc"),
                    src, "-o", str(exe)], check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "0 disagreements" in r.stdout
