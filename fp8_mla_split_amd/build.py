"""Build libmla.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m fp8_mla_split_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmla.so")
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into libmla.so; returns the library path."""
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU ops are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-inline-asm", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
        *srcs, "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
