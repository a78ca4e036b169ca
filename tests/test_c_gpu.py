"""The library used from plain C, with no Python binding and no torch
(needs an MI355X): tests/abi_consumer_gpu.c allocates with hipMalloc, runs a
grouped-query scan and a T4 decode step through include/gdn.h, and checks
them against the oracle within the tolerance and the scan against chained
decode launches bit for bit; then the one-launch decode step against its
stand-alone kernels and the split fused layer (workspace zeroed with
hipMemset) against the one-workgroup layer, bit for bit. __graft_entry__.build() links it into
tests/_bin/."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_bin", "abi_consumer_gpu")


def test_c_consumer_on_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(EXE):
        # a missing build output is reported, not failed, so that the runs
        # that stop at the first failure still reach the other GPU tests
        pytest.skip(f"{EXE} is not built: run __graft_entry__.build() first")
    print("running", EXE, flush=True)
    run = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-2000:]
    assert run.stdout.strip().endswith("0 failures")
