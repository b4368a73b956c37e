"""The library's host side under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/host/abi_checks.cpp drives every entry point of the C ABI (argument checks, calls that
pass them, a sweep of the split planner) against the library's host sources (the API and the
no-allocation entry point) and
tests/host/launch_stubs.cpp, which stands in for the kernel launchers; the sanitizers
instrument host code only (each -fsanitize flag is bound to the host pass), so nothing runs
on a GPU.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "abi_checks"
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "fp8_mla_split_amd", "csrc"),
           os.path.join(ROOT, "fp8_mla_split_amd", "csrc", "mla_api.hip"),
           os.path.join(ROOT, "fp8_mla_split_amd", "csrc", "noalloc.hip"),
           os.path.join(HERE, "host", "launch_stubs.cpp"),
           os.path.join(HERE, "host", "abi_checks.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    # the HIP runtime keeps allocations until exit by design; leak reports would be its own
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), \
        (res.stdout + res.stderr)[-3000:]
