"""Properties of the compiled gfx950 code, checked on the CPU from what the
compiler reports and emits (no GPU needed).

* Every kernel runs without scratch memory: no private stack, no register
  spills. A runtime-indexed private array or a spill lands in scratch, which
  the resource report shows even where a spill counter alone would not
  (the Foundry CUDA page asks the same of its warp kernels: a zero stack
  frame).
* The split decode layer's hand-off of y: each wave issues its device-scope
  y stores, then its state stores, then waits with an immediate vmcnt that
  leaves exactly those state stores in flight. Vector memory operations
  complete in issue order, so the wait covers the y stores only if exactly
  that many memory operations follow them before it. The test reads the
  locally built assembly of every instantiation and checks that sequence,
  so a compiler that splits, merges or reorders those stores is caught here
  rather than by a silent stale read on the GPU.
"""
import os
import re
import subprocess

import pytest

from linear_attention_ssm_recurrence_amd import build as hipbuild

REPORT = hipbuild.REPORT


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(REPORT):
        hipbuild.build()
    text = open(REPORT).read()
    kernels = {}
    name = None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
        if m and name:
            kernels[name][m.group(1).strip()] = m.group(2)
    return kernels


def test_every_kernel_has_no_scratch_and_no_spills(report):
    assert len(report) >= 90, f"only {len(report)} kernels in the resource report"
    bad = []
    for name, r in report.items():
        if (r.get("ScratchSize") != "0" or r.get("VGPRs Spill") != "0"
                or r.get("SGPRs Spill") != "0" or r.get("Dynamic Stack") != "False"):
            bad.append((name, r))
    assert not bad, f"kernels with scratch, spills or a dynamic stack: {bad[:3]}"


def test_report_names_the_hot_kernels(report):
    names = " ".join(report)
    for k in ("recurrence_decode_kernel", "recurrence_scan_kernel", "recurrence_short_scan_kernel",
              "decode_step_kernel", "decode_block_kernel", "decode_block_split_kernel",
              "chunk_prep_kernel", "chunk_scan_kernel", "prefill_frontend_kernel",
              "conv_scan_kernel", "conv_step_kernel", "gated_rmsnorm_d128_kernel"):
        assert k in names, k


VMEM = re.compile(r"^\s*(global|buffer|flat|scratch)_(load|store|atomic)\w*")


@pytest.fixture(scope="module")
def split_asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "gdn_block.s")
    cmd = hipbuild.asm_command(os.path.join(hipbuild.CSRC, "gdn_block.hip"))
    cmd[-1] = out
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    text = open(out).read()
    bodies = {}
    for m in re.finditer(r"^(_ZN3gdn25decode_block_split_kernel\w+):", text, re.M):
        end = text.index("s_endpgm", m.end())
        bodies[m.group(1)] = text[m.end():end].splitlines()
    return bodies


def test_split_layer_waits_for_its_y_stores(split_asm):
    """In each of the nine split-layer kernels: the y stores (dword, sc1),
    then exactly the wave's state stores (IT*E/4 = 4 float4 non-temporal
    stores), then `s_waitcnt vmcnt(4)`, with no other memory operation in
    between."""
    assert len(split_asm) == 9, sorted(split_asm)
    for name, lines in split_asm.items():
        first = next(i for i, l in enumerate(lines)
                     if re.match(r"^\s*global_store_dword\s.*\bsc1\b", l))
        ops, wait = [], None
        for l in lines[first:]:
            m = re.match(r"^\s*s_waitcnt\s+.*vmcnt\((\d+)\)", l)
            if m:
                wait = int(m.group(1))
                break
            if VMEM.match(l):
                ops.append(l.strip())
        y = [o for o in ops if re.match(r"global_store_dword\s.*\bsc1\b", o)]
        rest = ops[len(y):]
        assert ops[:len(y)] == y and len(y) >= 1, f"{name}: y stores not first: {ops}"
        assert wait == 4, f"{name}: wait vmcnt({wait}), expected 4"
        assert len(rest) == wait, f"{name}: {len(rest)} memory operations after the y stores: {rest}"
        assert all(re.match(r"global_store_dwordx4\s.*\bnt\b", o) for o in rest), rest
