"""CPU checks of host-side arithmetic that the kernels depend on."""
import os
import subprocess

import pytest

from conftest import ROOT


def test_fastdiv_constants_divide_exactly(tmp_path):
    """Every row mapping divides a flat index by a row length with a
    multiply-high constant prepared on the host; the constants must give the
    exact quotient for all indices below 2^31, for any divisor up to 2^30."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "fastdiv_check")
    src = os.path.join(ROOT, "tests", "fastdiv_check.hip")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), src,
                    "-o", exe], check=True, capture_output=True, timeout=600)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert ", 0 wrong" in r.stdout
