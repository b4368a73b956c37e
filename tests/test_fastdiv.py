"""Launch-time integer division helper (host logic of the decode launch), checked against
plain division on the CPU.  Compiles tests/fastdiv_check.cpp against the library's internal
header with hipcc and runs its host code."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_fast_div_matches_integer_division(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "fastdiv_check"
    subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I",
                    os.path.join(ROOT, "fp8_mla_split_amd", "csrc"), "-I",
                    os.path.join(ROOT, "include"), os.path.join(HERE, "fastdiv_check.cpp"),
                    "-o", str(exe)], check=True, capture_output=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
