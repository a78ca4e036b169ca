"""AddressSanitizer + UndefinedBehaviorSanitizer builds of host C code, on
the CPU:

* the oracle (oracle/gdn_oracle.c, float build) with a driver,
  tests/oracle_sanitize.c, that calls every routine on small inputs and at
  the edge sizes (one token, conv widths 1 to 65, ragged heads);
* tests/abi_consumer.c, the plain C caller of the library's argument checks,
  built as C11 and linked with libgdn.so.

Any out-of-bounds access, use of freed memory or undefined behaviour aborts
the run (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _gcc():
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no host compiler")
    return cc


def _run(exe, env=None):
    e = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
             UBSAN_OPTIONS="print_stacktrace=1")
    e.update(env or {})
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=e)


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = [_gcc(), "-std=c11", "-O1", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", *SAN,
           os.path.join(ROOT, "oracle", "gdn_oracle.c"), os.path.join(HERE, "oracle_sanitize.c"),
           "-o", exe, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    run = _run(exe)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "oracle sanitizer run: ok" in run.stdout


def test_abi_consumer_under_asan_ubsan(tmp_path):
    from linear_attention_ssm_recurrence_amd import build as hipbuild
    from linear_attention_ssm_recurrence_amd import gdn
    if not os.path.exists(gdn.LIB_PATH):
        hipbuild.build()
    libdir = os.path.dirname(gdn.LIB_PATH)
    exe = str(tmp_path / "abi_consumer_san")
    cmd = [_gcc(), "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", *SAN,
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_consumer.c"),
           "-L", libdir, "-lgdn", f"-Wl,-rpath,{libdir}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    # the HIP runtime keeps allocations for the life of the process: leaks are not checked here
    run = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert run.stdout.strip().endswith("0 failures"), run.stdout
