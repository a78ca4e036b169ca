"""Build the HIP library ``libgdn.so`` for gfx950 with hipcc.

Every kernel is compiled with packed-FP32 instructions disabled
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless. The per-kernel resource report
(VGPRs, SGPRs, scratch, LDS, occupancy) that ``-Rpass-analysis`` prints is
kept beside the library as ``libgdn.resource-usage.txt``.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn.so")
REPORT = os.path.join(PKG, "libgdn.resource-usage.txt")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def command(out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Rpass-analysis=kernel-resource-usage",
            "-I", INCLUDE, "-I", CSRC, *sources(), "-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ into libgdn.so; returns its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    with open(REPORT, "w") as f:
        f.write(" ".join(cmd) + "\n")
        f.write(res.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
