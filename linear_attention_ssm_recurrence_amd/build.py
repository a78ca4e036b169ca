"""Build the HIP library ``libgdn.so`` for gfx950 with hipcc, and the
benchmark's measurement probe ``libgdn_probe.so`` beside it.

Every kernel is compiled with packed-FP32 instructions disabled
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless. Each source under ``csrc/`` is
compiled to its own object (in parallel), then the objects are linked. The
per-kernel resource report (VGPRs, SGPRs, scratch, LDS, occupancy) that
``-Rpass-analysis`` prints is kept beside the library as
``libgdn.resource-usage.txt``. With ``keep_asm=True`` the gfx950 assembly of
each source is also written to ``_build/`` (for inspection by the tests).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROBE = os.path.join(PKG, "probe")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
PROBE_LIB = os.path.join(PKG, "libgdn_probe.so")
REPORT = os.path.join(PKG, "libgdn.resource-usage.txt")
ARCH = "gfx950"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _obj(src: str) -> str:
    return os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")


def compile_command(src: str) -> list[str]:
    return [hipcc(), *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", INCLUDE, "-I", CSRC,
            "-c", src, "-o", _obj(src)]


def asm_command(src: str) -> list[str]:
    out = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".gfx950.s")
    return [hipcc(), *FLAGS, "--cuda-device-only", "-S", "-I", INCLUDE, "-I", CSRC, src,
            "-o", out]


def _run(cmd: list[str], verbose: bool) -> subprocess.CompletedProcess:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")
    return res


def build(verbose: bool = False, keep_asm: bool = False, jobs: int = 8) -> str:
    """Compile every source under csrc/ into libgdn.so (and the probe into
    libgdn_probe.so); returns the path of libgdn.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    cmds = [compile_command(s) for s in srcs]
    if keep_asm:
        cmds += [asm_command(s) for s in srcs]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[_obj(s) for s in srcs],
          "-o", tmp], verbose)
    os.replace(tmp, LIB)
    with open(REPORT, "w") as f:
        for cmd, res in zip(cmds, results):
            if "-c" in cmd:
                f.write(" ".join(cmd) + "\n")
                f.write(res.stderr)
    ptmp = PROBE_LIB + ".tmp"
    _run([hipcc(), *FLAGS, "-shared", "-I", PROBE, os.path.join(PROBE, "gdn_probe.hip"),
          "-o", ptmp], verbose)
    os.replace(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
