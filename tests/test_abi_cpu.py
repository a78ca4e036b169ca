"""The C-ABI library on the host: it loads, exports every symbol gdn.h
declares, and rejects bad arguments before launching anything.

No call here reaches a kernel launch: every argument set fails validation (or
is an empty input, which returns before any HIP call), so these tests need no
GPU and are safe on one.
"""
import ctypes
import os
import re

import pytest

from linear_attention_ssm_recurrence_amd import build as hipbuild
from linear_attention_ssm_recurrence_amd import gdn

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p(0x10004)    # not 16-byte aligned, never dereferenced
NUL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        hipbuild.build()
    return gdn.load_library()


def test_exports_every_header_symbol(lib):
    names = gdn.header_symbols()
    assert len(names) == 24, names
    out = os.popen(f"nm -D --defined-only {gdn.LIB_PATH}").read()
    exported = set(re.findall(r"\sT\s(gdn_\w+)", out))
    for name in names:
        assert name in exported, f"{name} declared in gdn.h but not exported"
        assert hasattr(lib, name)


@pytest.mark.parametrize("std", ["c11", "c++17"])
def test_c_consumer(lib, tmp_path, std):
    """tests/abi_consumer.c, a plain C caller, builds as strict C11 and as
    C++17 against include/gdn.h, links against
    libgdn.so (every declared function must resolve), and gets the expected
    code from each entry point's argument checks through the header's own
    prototypes. None of its calls passes validation, so nothing is launched."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if std == "c11" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    here = os.path.dirname(os.path.abspath(__file__))
    include = os.path.join(os.path.dirname(here), "include")
    libdir = os.path.dirname(gdn.LIB_PATH)
    exe = str(tmp_path / f"abi_consumer_{std.replace('+', 'p')}")
    src = os.path.join(here, "abi_consumer.c")
    cmd = [cc, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", include]
    cmd += (["-x", "c++"] if std.startswith("c++") else []) + [src]
    cmd += ["-L", libdir, "-lgdn", f"-Wl,-rpath,{libdir}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-2000:]
    assert run.stdout.strip().endswith("0 failures"), run.stdout


def test_version_and_strerror(lib):
    assert lib.gdn_abi_version() == 1
    for code in range(6):
        assert gdn.strerror(code)
    assert "unknown" in gdn.strerror(99)


def rec(lib, state=FAKE, q=FAKE, k=FAKE, n_seqs=1, H=2, S=32, seq=False, T=1):
    f = lib.gdn_recurrence_seq if seq else lib.gdn_recurrence
    args = [state, q, k, FAKE, FAKE, FAKE, FAKE, n_seqs] + ([T] if seq else []) + [H, S, 1.0, NUL]
    return f(*args)


@pytest.mark.parametrize("seq", [False, True])
def test_recurrence_validation(lib, seq):
    assert rec(lib, state=NUL, seq=seq) == gdn.GDN_ENULL
    assert rec(lib, n_seqs=-1, seq=seq) == gdn.GDN_ESIZE
    assert rec(lib, H=0, seq=seq) == gdn.GDN_ESIZE
    assert rec(lib, S=0, seq=seq) == gdn.GDN_ESIZE
    for bad_s in (16, 48, 96, 512):
        assert rec(lib, S=bad_s, seq=seq) == gdn.GDN_EUNSUPPORTED
    assert rec(lib, state=FAKE_MIS, seq=seq) == gdn.GDN_EALIGN
    assert rec(lib, q=FAKE_MIS, seq=seq) == gdn.GDN_EALIGN
    # bad shape wins over a NULL pointer
    assert rec(lib, state=NUL, S=48, seq=seq) == gdn.GDN_EUNSUPPORTED
    # empty inputs: no work, pointers not inspected
    assert rec(lib, state=NUL, q=NUL, k=NUL, n_seqs=0, seq=seq) == gdn.GDN_OK
    if seq:
        assert rec(lib, T=0, seq=True) == gdn.GDN_OK
        assert rec(lib, T=-3, seq=True) == gdn.GDN_ESIZE
    # sizes whose flattened element count overflows the library's limit
    assert rec(lib, n_seqs=2**30, H=2**20, S=256, seq=seq) == gdn.GDN_ESIZE


@pytest.mark.parametrize("fn", ["gdn_conv1d_silu", "gdn_conv1d_silu_seq"])
def test_conv_validation(lib, fn):
    f = getattr(lib, fn)
    seq = fn.endswith("_seq")

    def call(x=FAKE, n=1, T=1, C=8, K=4):
        args = [x, FAKE, FAKE, FAKE, n] + ([T] if seq else []) + [C, K, NUL]
        return f(*args)

    assert call(x=NUL) == gdn.GDN_ENULL
    assert call(n=-1) == gdn.GDN_ESIZE
    assert call(C=0) == gdn.GDN_ESIZE
    assert call(K=0) == gdn.GDN_ESIZE
    for K in (1, 5, 8):
        assert call(K=K) == gdn.GDN_EUNSUPPORTED
    assert call(x=NUL, n=0) == gdn.GDN_OK
    if seq:
        assert call(T=-1) == gdn.GDN_ESIZE
        assert call(x=NUL, T=0) == gdn.GDN_OK


def test_pointwise_validation(lib):
    assert lib.gdn_decay_gate(NUL, FAKE, FAKE, FAKE, 4, 1, NUL) == gdn.GDN_ENULL
    assert lib.gdn_decay_gate(FAKE, FAKE, FAKE, FAKE, 0, 1, NUL) == gdn.GDN_ESIZE
    assert lib.gdn_decay_gate(FAKE, FAKE, FAKE, FAKE, 4, -1, NUL) == gdn.GDN_ESIZE
    assert lib.gdn_decay_gate(NUL, NUL, NUL, NUL, 4, 0, NUL) == gdn.GDN_OK
    assert lib.gdn_sigmoid(NUL, FAKE, 3, NUL) == gdn.GDN_ENULL
    assert lib.gdn_sigmoid(FAKE, FAKE, -3, NUL) == gdn.GDN_ESIZE
    assert lib.gdn_sigmoid(NUL, NUL, 0, NUL) == gdn.GDN_OK
    l2 = lib.gdn_l2norm_gqa
    assert l2(NUL, FAKE, 1, 2, 4, 32, 1e-6, NUL) == gdn.GDN_ENULL
    assert l2(FAKE, FAKE, 1, 3, 4, 32, 1e-6, NUL) == gdn.GDN_ESIZE      # 4 % 3 != 0
    assert l2(FAKE, FAKE, 1, 2, 4, 30, 1e-6, NUL) == gdn.GDN_EUNSUPPORTED
    assert l2(FAKE, FAKE, 1, 2, 4, 2048, 1e-6, NUL) == gdn.GDN_EUNSUPPORTED
    assert l2(FAKE_MIS, FAKE, 1, 2, 4, 32, 1e-6, NUL) == gdn.GDN_EALIGN
    assert l2(NUL, NUL, 0, 2, 4, 32, 1e-6, NUL) == gdn.GDN_OK
    nm = lib.gdn_gated_rmsnorm
    assert nm(FAKE, NUL, FAKE, FAKE, 1, 32, 1e-6, NUL) == gdn.GDN_ENULL
    assert nm(FAKE, FAKE, FAKE, FAKE, -1, 32, 1e-6, NUL) == gdn.GDN_ESIZE
    assert nm(FAKE, FAKE, FAKE, FAKE, 1, 0, 1e-6, NUL) == gdn.GDN_ESIZE
    assert nm(FAKE, FAKE, FAKE, FAKE, 1, 34, 1e-6, NUL) == gdn.GDN_EUNSUPPORTED
    assert nm(FAKE, FAKE, FAKE_MIS, FAKE, 1, 32, 1e-6, NUL) == gdn.GDN_EALIGN
    assert nm(NUL, NUL, NUL, NUL, 0, 32, 1e-6, NUL) == gdn.GDN_OK


def test_ex_validation(lib):
    f = lib.gdn_recurrence_ex

    def rex(HK=2, H=4, S=32, variant=0, state=FAKE, n=1):
        return f(state, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n, HK, H, S, 1.0, variant, NUL)

    assert rex(variant=2) == gdn.GDN_EUNSUPPORTED
    assert rex(variant=-1) == gdn.GDN_EUNSUPPORTED
    assert rex(HK=3) == gdn.GDN_ESIZE
    assert rex(HK=0) == gdn.GDN_ESIZE
    assert rex(state=NUL) == gdn.GDN_ENULL
    assert rex(state=NUL, n=0) == gdn.GDN_OK
    fs = lib.gdn_recurrence_seq_ex

    def rsx(snaps=NUL, HK=2, T=3, n=1, variant=gdn.GDN_RECUR_EXACT):
        return fs(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, snaps, n, T, HK, 4, 32, 1.0, variant,
                  NUL)

    assert rsx(variant=2) == gdn.GDN_EUNSUPPORTED
    assert rsx(variant=-1, n=0) == gdn.GDN_EUNSUPPORTED    # checked before anything else
    assert rsx(variant=gdn.GDN_RECUR_T4, T=0) == gdn.GDN_OK
    assert rsx(snaps=FAKE_MIS) == gdn.GDN_EALIGN
    assert rsx(HK=3) == gdn.GDN_ESIZE
    assert rsx(T=-1) == gdn.GDN_ESIZE
    assert rsx(T=0) == gdn.GDN_OK
    fc = lib.gdn_conv1d_silu_seq_ex
    assert fc(FAKE, FAKE, FAKE, FAKE, NUL, 1, 1, 8, 5, NUL) == gdn.GDN_EUNSUPPORTED
    assert fc(NUL, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 4, NUL) == gdn.GDN_ENULL


def test_block_validation(lib):
    f = lib.gdn_decode_block_bf16

    def call(first=FAKE, state=FAKE, n=1, HK=16, H=32, S=128, K=4, z=FAKE):
        return f(first, z, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, state, FAKE,
                 n, HK, H, S, K, 0.1, 1e-6, 1e-6, NUL)

    assert call(first=NUL) == gdn.GDN_ENULL
    assert call(n=-1) == gdn.GDN_ESIZE
    assert call(HK=0) == gdn.GDN_ESIZE
    assert call(HK=12) == gdn.GDN_ESIZE                 # 32 % 12 != 0
    assert call(HK=4) == gdn.GDN_EUNSUPPORTED           # 8 V-heads per K-head
    assert call(S=64) == gdn.GDN_EUNSUPPORTED
    assert call(K=5) == gdn.GDN_EUNSUPPORTED
    assert call(state=FAKE_MIS) == gdn.GDN_EALIGN
    assert call(z=ctypes.c_void_p(0x10002)) == gdn.GDN_EALIGN
    assert call(first=NUL, state=NUL, n=0) == gdn.GDN_OK


def test_block_noalloc_validation(lib):
    """The allocation-free split layer checks its arguments as the workspace
    form does, and refuses with GDN_ESIZE a batch whose counters
    (n_seqs * (n_k_heads + n_v_heads)) exceed its array, before it looks up
    the array or launches anything."""
    f = lib.gdn_decode_block_bf16_noalloc

    def call(first=FAKE, state=FAKE, n=3, HK=16, H=32, S=128, K=4, z=FAKE):
        return f(first, z, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, state, FAKE,
                 n, HK, H, S, K, 0.1, 1e-6, 1e-6, NUL)

    cap = gdn.GDN_NOALLOC_MAX_COUNTERS
    assert cap == 65536
    assert call(n=cap // 48 + 1) == gdn.GDN_ESIZE       # 1366 x (16 + 32) > 65536
    assert call(first=NUL) == gdn.GDN_ENULL
    assert call(n=-1) == gdn.GDN_ESIZE
    assert call(HK=12) == gdn.GDN_ESIZE
    assert call(HK=4) == gdn.GDN_EUNSUPPORTED
    assert call(S=64) == gdn.GDN_EUNSUPPORTED
    assert call(K=5) == gdn.GDN_EUNSUPPORTED
    assert call(state=FAKE_MIS) == gdn.GDN_EALIGN
    assert call(z=ctypes.c_void_p(0x10002)) == gdn.GDN_EALIGN
    assert call(first=NUL, state=NUL, n=0) == gdn.GDN_OK


def test_decode_step_validation(lib):
    f = lib.gdn_decode_step

    def call(state=FAKE, q=FAKE, a=FAKE, n=2, HK=16, H=32, S=128):
        return f(state, q, FAKE, FAKE, a, FAKE, FAKE, FAKE, FAKE, n, HK, H, S, 0.1, 1e-6, NUL)

    assert call(a=NUL) == gdn.GDN_ENULL
    assert call(state=NUL) == gdn.GDN_ENULL
    assert call(n=-1) == gdn.GDN_ESIZE
    assert call(HK=0) == gdn.GDN_ESIZE
    assert call(HK=12) == gdn.GDN_ESIZE                 # 32 % 12 != 0
    assert call(S=96) == gdn.GDN_EUNSUPPORTED
    assert call(state=FAKE_MIS) == gdn.GDN_EALIGN
    assert call(q=FAKE_MIS) == gdn.GDN_EALIGN
    assert call(state=NUL, q=NUL, a=NUL, n=0) == gdn.GDN_OK


def test_block_ex_validation(lib):
    f = lib.gdn_decode_block_bf16_ex
    need = lib.gdn_decode_block_workspace_bytes(3, 16, 32)
    assert need == (3 * 16 + 3 * 32) * 4
    assert lib.gdn_decode_block_workspace_bytes(3, 16, 24) == 0   # 24 % 16 != 0
    assert lib.gdn_decode_block_workspace_bytes(3, 0, 32) == 0
    assert lib.gdn_decode_block_workspace_bytes(-1, 16, 32) == 0
    assert lib.gdn_decode_block_workspace_bytes(0, 16, 32) == 0

    def call(first=FAKE, state=FAKE, ws=FAKE, ws_bytes=need, n=3, HK=16, H=32, S=128, K=4,
             z=FAKE):
        return f(first, z, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, state, FAKE, ws, ws_bytes,
                 n, HK, H, S, K, 0.1, 1e-6, 1e-6, NUL)

    assert call(first=NUL) == gdn.GDN_ENULL
    assert call(ws=NUL) == gdn.GDN_ENULL
    assert call(ws_bytes=need - 1) == gdn.GDN_ESIZE
    assert call(ws=ctypes.c_void_p(0x10002)) == gdn.GDN_EALIGN
    assert call(n=-1) == gdn.GDN_ESIZE
    assert call(HK=12) == gdn.GDN_ESIZE                 # 32 % 12 != 0
    assert call(HK=4) == gdn.GDN_EUNSUPPORTED           # 8 V-heads per K-head
    assert call(S=64) == gdn.GDN_EUNSUPPORTED
    assert call(K=1) == gdn.GDN_EUNSUPPORTED
    assert call(state=FAKE_MIS) == gdn.GDN_EALIGN
    assert call(z=ctypes.c_void_p(0x10002)) == gdn.GDN_EALIGN
    assert call(first=NUL, state=NUL, ws=NUL, n=0) == gdn.GDN_OK


def test_prefill_validation(lib):
    f = lib.gdn_prefill_bf16
    need = lib.gdn_prefill_workspace_bytes(1, 8, 2, 4, 128)
    assert need > 0
    assert lib.gdn_prefill_workspace_bytes(1, 8, 2, 4, 0) == 0

    def call(first=FAKE, ws=FAKE, ws_bytes=need, n=1, T=8, HK=2, H=4, S=128, K=4):
        return f(first, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes,
                 n, T, HK, H, S, K, 0.1, 1e-6, 1e-6, NUL)

    assert call(first=NUL) == gdn.GDN_ENULL
    assert call(ws=NUL) == gdn.GDN_ENULL
    assert call(ws_bytes=need - 1) == gdn.GDN_ESIZE
    assert call(ws=ctypes.c_void_p(0x10010)) == gdn.GDN_EALIGN
    assert call(HK=3) == gdn.GDN_ESIZE
    assert call(S=64) == gdn.GDN_EUNSUPPORTED
    assert call(K=1) == gdn.GDN_EUNSUPPORTED
    assert call(T=-1) == gdn.GDN_ESIZE
    assert call(first=NUL, ws=NUL, T=0) == gdn.GDN_OK


def test_probe_is_not_in_the_library(lib):
    """The benchmark's FMA probe lives in its own library, libgdn_probe.so,
    not among libgdn.so's exports; its argument checks return before any
    launch."""
    out = os.popen(f"nm -D --defined-only {gdn.LIB_PATH}").read()
    assert "gdn_probe_fma" not in out
    path = os.path.join(os.path.dirname(gdn.LIB_PATH), "libgdn_probe.so")
    probe = ctypes.CDLL(path)
    f = probe.gdn_probe_fma
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(FAKE, 0, 10, 1.0, 0.0, NUL) == 2
    assert f(FAKE, 4, 0, 1.0, 0.0, NUL) == 2
    assert f(FAKE, (1 << 20) + 1, 10, 1.0, 0.0, NUL) == 2
    assert f(NUL, 4, 10, 1.0, 0.0, NUL) == 1
    m = probe.gdn_probe_mfma
    m.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    m.restype = ctypes.c_int
    assert m(0, 3, FAKE, 4, 10, NUL) == 3
    assert m(2, 1, FAKE, 4, 10, NUL) == 3
    assert m(0, 1, NUL, 4, 10, NUL) == 1
    assert m(1, 2, FAKE, 0, 10, NUL) == 2


def test_ssm_a_validation(lib):
    f = lib.gdn_ssm_a
    assert f(NUL, FAKE, 4, NUL) == gdn.GDN_ENULL
    assert f(FAKE, NUL, 4, NUL) == gdn.GDN_ENULL
    assert f(FAKE, FAKE, -1, NUL) == gdn.GDN_ESIZE
    assert f(NUL, NUL, 0, NUL) == gdn.GDN_OK


def test_prefill_checks_the_scan_before_launching(lib):
    """A prefill whose chunked scan would exceed its grid limit (8 blocks per
    (sequence, V-head): 2^22 sequences x 64 heads) is refused with GDN_ESIZE
    before the front end (which rolls conv_state in place) is launched: a
    launch on this host, which has no GPU, would have returned GDN_ELAUNCH."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("argument-check test for a host without a GPU")
    N, T, HK, H = 1 << 22, 1, 64, 64
    args = [FAKE] * 11 + [FAKE, ctypes.c_size_t(1 << 62), N, T, HK, H, 128, 4, 0.1, 1e-6, 1e-6]
    assert lib.gdn_prefill_bf16_ex(*args, gdn.GDN_SCAN_CHUNKED, NUL) == gdn.GDN_ESIZE


def test_prefill_ex_validation(lib):
    f = lib.gdn_prefill_bf16_ex
    need = lib.gdn_prefill_workspace_bytes(1, 100, 2, 4, 128)
    assert need >= lib.gdn_chunked_workspace_bytes(1, 100, 4, 128)

    def call(first=FAKE, ws=FAKE, ws_bytes=need, T=100, S=128, scan=gdn.GDN_SCAN_CHUNKED):
        return f(first, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes,
                 1, T, 2, 4, S, 4, 0.1, 1e-6, 1e-6, scan, NUL)

    assert call(scan=2) == gdn.GDN_EUNSUPPORTED
    assert call(scan=-1) == gdn.GDN_EUNSUPPORTED
    assert call(first=NUL) == gdn.GDN_ENULL
    assert call(ws_bytes=need - 1) == gdn.GDN_ESIZE
    assert call(S=64) == gdn.GDN_EUNSUPPORTED
    assert call(first=NUL, ws=NUL, T=0, scan=gdn.GDN_SCAN_SEQUENTIAL) == gdn.GDN_OK


def test_chunked_validation(lib):
    f = lib.gdn_recurrence_seq_chunked
    need = lib.gdn_chunked_workspace_bytes(1, 100, 4, 128)
    assert need == 1 * 4 * 2 * 8448 * 4
    assert lib.gdn_chunked_workspace_bytes(1, 100, 4, 64) == 0

    def call(state=FAKE, ws=FAKE, ws_bytes=need, T=100, HK=2, H=4, S=128, y=FAKE):
        return f(state, FAKE, FAKE, FAKE, FAKE, FAKE, y, ws, ws_bytes, 1, T, HK, H, S, 0.1, NUL)

    assert call(state=NUL) == gdn.GDN_ENULL
    assert call(ws=NUL) == gdn.GDN_ENULL
    assert call(ws_bytes=need - 4) == gdn.GDN_ESIZE
    assert call(S=64) == gdn.GDN_EUNSUPPORTED
    assert call(HK=3) == gdn.GDN_ESIZE
    assert call(state=FAKE_MIS) == gdn.GDN_EALIGN
    assert call(ws=FAKE_MIS) == gdn.GDN_EALIGN
    assert call(y=FAKE_MIS) == gdn.GDN_EALIGN
    assert call(state=NUL, ws=NUL, T=0) == gdn.GDN_OK


def test_python_binding_rejects_cpu_tensors(lib):
    import torch
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        gdn.gdn_sigmoid(x, x)


def test_python_binding_validation(lib):
    """The binding checks shapes, devices and types before it calls the
    library: a wrong shape or a CPU tensor raises ValueError, a non-tensor
    TypeError, and nothing reaches the library (no GPU is needed here)."""
    import torch
    N, T, HK, H, S = 2, 3, 2, 4, 32
    st = torch.zeros(N, H, S, S)
    qh = torch.zeros(N, HK, S)
    v = torch.zeros(N, H, S)
    g = torch.zeros(N, H)
    y = torch.zeros(N, H, S)
    # shapes (checked first)
    with pytest.raises(ValueError, match="state"):
        gdn.gdn_recurrence_ex(torch.zeros(N, H, S, S + 1), qh, qh, v, g, g, y, 1.0)
    with pytest.raises(ValueError, match="y"):
        gdn.gdn_recurrence_ex(st, qh, qh, v, g, g, torch.zeros(N, H, S + 1), 1.0)
    qs = torch.zeros(N, T, HK, S)
    vs = torch.zeros(N, T, H, S)
    gs = torch.zeros(N, T, H)
    with pytest.raises(ValueError, match="snaps"):
        gdn.gdn_recurrence_seq_ex(st, qs, qs, vs, gs, gs, vs.clone(), 1.0,
                                  snaps=torch.zeros(N, T, H, S, S + 1))
    with pytest.raises(ValueError, match="g"):
        gdn.gdn_recurrence_seq_ex(st, qs, qs, vs, torch.zeros(N, T, H + 1), gs, vs.clone(), 1.0)
    with pytest.raises(ValueError):
        gdn.gdn_conv1d_silu_seq(torch.zeros(N, T, 8), torch.zeros(8, 4), torch.zeros(N, 8, 2),
                                torch.zeros(N, T, 8))
    with pytest.raises(ValueError):
        gdn.gdn_gated_rmsnorm(torch.zeros(5, 32), torch.zeros(31), torch.zeros(5, 32),
                              torch.zeros(5, 32))
    with pytest.raises(ValueError, match="conv_dim"):
        C, K = 2 * 16 * 128 + 32 * 128, 4
        gdn.gdn_decode_block_bf16(torch.zeros(1, C + 8, dtype=torch.int16),
                                  torch.zeros(1, 32, 128, dtype=torch.int16), torch.zeros(1, 32),
                                  torch.zeros(1, 32), torch.zeros(C + 8, K), torch.zeros(32),
                                  torch.zeros(32), torch.zeros(128), torch.zeros(1, C + 8, K - 1),
                                  torch.zeros(1, 32, 128, 128), torch.zeros(1, 32, 128), 16, 0.1)
    # devices and types (shapes right)
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gdn_recurrence_ex(st, qh, qh, v, g, g, y, 1.0)
    with pytest.raises(ValueError, match="GPU tensor"):
        ws = torch.zeros(gdn.gdn_chunked_workspace_bytes(N, T, H, 128), dtype=torch.uint8)
        st128, q128, v128 = torch.zeros(N, H, 128, 128), torch.zeros(N, T, HK, 128), torch.zeros(N, T, H, 128)
        gdn.gdn_recurrence_seq_chunked(st128, q128, q128, v128, gs, gs, v128.clone(), 1.0, ws)
    with pytest.raises(TypeError):
        gdn.gdn_sigmoid([0.0, 1.0], torch.zeros(2))
    with pytest.raises(ValueError, match="same device"):
        gdn.gdn_sigmoid(torch.zeros(2), torch.zeros(2, device="meta"))
