"""Python binding of the C ABI in ``include/gdn.h`` (``libgdn.so``).

Argument marshalling only: each function checks that the tensors are on the
GPU with the expected dtype, shape and contiguity, passes their device pointers
and sizes to the entry point of the same name, and raises ``GdnError`` on a
non-zero return code. Every step of the computation runs in the HIP kernels;
nothing here computes. The work is enqueued on the current torch stream of the
tensors' device (or on ``stream`` when given) and the functions return without
synchronising.

If ``libgdn.so`` has not been built, importing the library raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import functools
import glob
import numbers
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "gdn.h")

GDN_OK, GDN_ENULL, GDN_ESIZE, GDN_EUNSUPPORTED, GDN_EALIGN, GDN_ELAUNCH = range(6)
GDN_RECUR_EXACT, GDN_RECUR_T4 = 0, 1
GDN_SCAN_SEQUENTIAL, GDN_SCAN_CHUNKED = 0, 1
GDN_NOALLOC_MAX_COUNTERS = 65536


class GdnError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {text} (code {code})")
        self.code = code


_lib = None


def load_library():
    """Load libgdn.so and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    sig = {
        "gdn_decay_gate": [P, P, P, P, I, L, P],
        "gdn_sigmoid": [P, P, L, P],
        "gdn_l2norm_gqa": [P, P, L, I, I, I, F, P],
        "gdn_conv1d_silu": [P, P, P, P, I, I, I, P],
        "gdn_conv1d_silu_seq": [P, P, P, P, I, I, I, I, P],
        "gdn_recurrence": [P, P, P, P, P, P, P, I, I, I, F, P],
        "gdn_recurrence_ex": [P, P, P, P, P, P, P, I, I, I, I, F, I, P],
        "gdn_decode_step": [P] * 9 + [I, I, I, I, F, F, P],
        "gdn_recurrence_seq_ex": [P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, P],
        "gdn_conv1d_silu_seq_ex": [P, P, P, P, P, I, I, I, I, P],
        "gdn_recurrence_seq": [P, P, P, P, P, P, P, I, I, I, I, F, P],
        "gdn_gated_rmsnorm": [P, P, P, P, L, I, F, P],
        "gdn_decode_block_bf16": [P] * 11 + [I] * 5 + [F] * 3 + [P],
        "gdn_decode_block_bf16_ex": [P] * 12 + [ctypes.c_size_t] + [I] * 5 + [F] * 3 + [P],
        "gdn_decode_block_bf16_noalloc": [P] * 11 + [I] * 5 + [F] * 3 + [P],
        "gdn_prefill_bf16": [P] * 12 + [ctypes.c_size_t] + [I] * 6 + [F] * 3 + [P],
        "gdn_prefill_bf16_ex": [P] * 12 + [ctypes.c_size_t] + [I] * 6 + [F] * 3 + [I, P],
        "gdn_recurrence_seq_chunked": [P] * 8 + [ctypes.c_size_t] + [I] * 5 + [F, P],
        "gdn_ssm_a": [P, P, I, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = I
    lib.gdn_strerror.argtypes = [I]
    lib.gdn_strerror.restype = ctypes.c_char_p
    lib.gdn_abi_version.restype = I
    lib.gdn_prefill_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.gdn_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_chunked_workspace_bytes.argtypes = [I, I, I, I]
    lib.gdn_chunked_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_decode_block_workspace_bytes.argtypes = [I, I, I]
    lib.gdn_decode_block_workspace_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def header_symbols() -> list[str]:
    """Names of the entry points declared in the headers under include/."""
    names = set()
    for path in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        text = open(path).read()
        names |= set(re.findall(r"^\s*(?:const\s+char\s*\*|int|size_t)\s*(gdn_\w+)\s*\(", text, re.M))
    return sorted(names)


def strerror(code: int) -> str:
    return load_library().gdn_strerror(int(code)).decode()


def _typed(fn):
    """Reject, with TypeError, any argument that is not a tensor, a number,
    None or a stream, and, with ValueError, tensors on different devices,
    before the function reads shapes from its arguments. The call then runs
    with the tensors' GPU as the current device, which is the device the
    library launches on."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        device = None
        for i, a in enumerate(list(args) + list(kwargs.values())):
            if isinstance(a, torch.Tensor):
                if device is None:
                    device = a.device
                elif a.device != device:
                    raise ValueError(f"{fn.__name__}: every tensor must be on the same device "
                                     f"(argument {i} is on {a.device}, an earlier one on {device})")
            elif not (isinstance(a, numbers.Number) or a is None or hasattr(a, "cuda_stream")):
                raise TypeError(f"{fn.__name__}: argument {i} must be a torch.Tensor or a "
                                f"number, got {type(a).__name__}")
        if (device is not None and device.type == "cuda" and device.index is not None
                and device.index != torch.cuda.current_device()):
            with torch.cuda.device(device):
                return fn(*args, **kwargs)
        return fn(*args, **kwargs)
    return wrapper


def _call(name: str, *args) -> None:
    rc = getattr(load_library(), name)(*args)
    if rc != GDN_OK:
        raise GdnError(name, rc, strerror(rc))


def _ptr(t: torch.Tensor, dtype, what: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a GPU tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _shape(t: torch.Tensor, shape: tuple, what: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")


F32 = torch.float32


@_typed
def gdn_ssm_a(A_log, ssm_a, stream=None):
    """ssm_a[h] = -exp(A_log[h]), the gate's per-head factor (prepared once
    per layer's parameters); A_log, ssm_a [H]."""
    H = A_log.numel()
    _shape(A_log, (H,), "A_log")
    _shape(ssm_a, (H,), "ssm_a")
    _call("gdn_ssm_a", _ptr(A_log, F32, "A_log"), _ptr(ssm_a, F32, "ssm_a"), H,
          _stream(A_log, stream))


@_typed
def gdn_decay_gate(a, dt_bias, ssm_a, g, stream=None):
    """g[..., h] = ssm_a[h] * softplus(a[..., h] + dt_bias[h]), ssm_a = -exp(A_log)."""
    H = ssm_a.shape[0]
    _shape(dt_bias, (H,), "dt_bias")
    _shape(g, a.shape, "g")
    _call("gdn_decay_gate", _ptr(a, F32, "a"), _ptr(dt_bias, F32, "dt_bias"),
          _ptr(ssm_a, F32, "ssm_a"), _ptr(g, F32, "g"), H, a.numel() // max(H, 1),
          _stream(a, stream))


@_typed
def gdn_sigmoid(x, y, stream=None):
    _shape(y, x.shape, "y")
    _call("gdn_sigmoid", _ptr(x, F32, "x"), _ptr(y, F32, "y"), x.numel(), _stream(x, stream))


@_typed
def gdn_l2norm_gqa(x, out, eps=1e-6, stream=None):
    """x [..., HK, D] -> out [..., H, D]; V-head vh reads K-head vh mod HK."""
    HK, D = x.shape[-2:]
    H = out.shape[-2]
    _shape(out, tuple(x.shape[:-2]) + (H, D), "out")
    rows = x.numel() // max(HK * D, 1)
    _call("gdn_l2norm_gqa", _ptr(x, F32, "x"), _ptr(out, F32, "out"), rows, HK, H, D,
          float(eps), _stream(x, stream))


@_typed
def gdn_conv1d_silu(x, w, conv_state, out, stream=None):
    """x, out [N][C]; w [C][K]; conv_state [N][C][K-1] updated in place."""
    N, C = x.shape
    K = w.shape[1]
    _shape(w, (C, K), "w")
    _shape(conv_state, (N, C, K - 1), "conv_state")
    _shape(out, (N, C), "out")
    _call("gdn_conv1d_silu", _ptr(x, F32, "x"), _ptr(w, F32, "w"), _ptr(conv_state, F32, "conv_state"),
          _ptr(out, F32, "out"), N, C, K, _stream(x, stream))


@_typed
def gdn_conv1d_silu_seq(x, w, conv_state, out, stream=None):
    """x, out [N][T][C]; w [C][K]; conv_state [N][C][K-1] updated in place."""
    N, T, C = x.shape
    K = w.shape[1]
    _shape(w, (C, K), "w")
    _shape(conv_state, (N, C, K - 1), "conv_state")
    _shape(out, (N, T, C), "out")
    _call("gdn_conv1d_silu_seq", _ptr(x, F32, "x"), _ptr(w, F32, "w"),
          _ptr(conv_state, F32, "conv_state"), _ptr(out, F32, "out"), N, T, C, K,
          _stream(x, stream))


@_typed
def gdn_recurrence(state, q, k, v, g, beta, y, scale, stream=None):
    """state [N][H][S][S] in place; q, k, v, y [N][H][S]; g, beta [N][H]."""
    N, H, S = q.shape
    _shape(state, (N, H, S, S), "state")
    for t, nm in ((k, "k"), (v, "v"), (y, "y")):
        _shape(t, (N, H, S), nm)
    _shape(g, (N, H), "g")
    _shape(beta, (N, H), "beta")
    _call("gdn_recurrence", _ptr(state, F32, "state"), _ptr(q, F32, "q"), _ptr(k, F32, "k"),
          _ptr(v, F32, "v"), _ptr(g, F32, "g"), _ptr(beta, F32, "beta"), _ptr(y, F32, "y"),
          N, H, S, float(scale), _stream(q, stream))


@_typed
def gdn_recurrence_seq(state, q, k, v, g, beta, y, scale, stream=None):
    """state [N][H][S][S] in place; q, k, v, y [N][T][H][S]; g, beta [N][T][H]."""
    N, T, H, S = q.shape
    _shape(state, (N, H, S, S), "state")
    for t, nm in ((k, "k"), (v, "v"), (y, "y")):
        _shape(t, (N, T, H, S), nm)
    _shape(g, (N, T, H), "g")
    _shape(beta, (N, T, H), "beta")
    _call("gdn_recurrence_seq", _ptr(state, F32, "state"), _ptr(q, F32, "q"), _ptr(k, F32, "k"),
          _ptr(v, F32, "v"), _ptr(g, F32, "g"), _ptr(beta, F32, "beta"), _ptr(y, F32, "y"),
          N, T, H, S, float(scale), _stream(q, stream))


@_typed
def gdn_recurrence_ex(state, q, k, v, g, beta, y, scale, variant=GDN_RECUR_EXACT, stream=None):
    """state [N][H][S][S] in place; q, k [N][HK][S] (V-head h reads K-head
    h mod HK); v, y [N][H][S]; g, beta [N][H]."""
    N, H, S = v.shape
    HK = q.shape[1]
    _shape(state, (N, H, S, S), "state")
    _shape(q, (N, HK, S), "q")
    _shape(k, (N, HK, S), "k")
    _shape(y, (N, H, S), "y")
    _shape(g, (N, H), "g")
    _shape(beta, (N, H), "beta")
    _call("gdn_recurrence_ex", _ptr(state, F32, "state"), _ptr(q, F32, "q"), _ptr(k, F32, "k"),
          _ptr(v, F32, "v"), _ptr(g, F32, "g"), _ptr(beta, F32, "beta"), _ptr(y, F32, "y"),
          N, HK, H, S, float(scale), int(variant), _stream(v, stream))


@_typed
def gdn_decode_step(state, q, k, v, a, b, ssm_a, dt_bias, y, scale, l2_eps=1e-6, stream=None):
    """One decode step from raw inputs: state [N][H][S][S] in place; q, k
    [N][HK][S] raw (normalised in the kernel); v, y [N][H][S]; a, b [N][H];
    ssm_a, dt_bias [H]."""
    N, H, S = v.shape
    HK = q.shape[1]
    _shape(state, (N, H, S, S), "state")
    _shape(q, (N, HK, S), "q")
    _shape(k, (N, HK, S), "k")
    _shape(y, (N, H, S), "y")
    _shape(a, (N, H), "a")
    _shape(b, (N, H), "b")
    _shape(ssm_a, (H,), "ssm_a")
    _shape(dt_bias, (H,), "dt_bias")
    _call("gdn_decode_step", _ptr(state, F32, "state"), _ptr(q, F32, "q"), _ptr(k, F32, "k"),
          _ptr(v, F32, "v"), _ptr(a, F32, "a"), _ptr(b, F32, "b"), _ptr(ssm_a, F32, "ssm_a"),
          _ptr(dt_bias, F32, "dt_bias"), _ptr(y, F32, "y"), N, HK, H, S, float(scale),
          float(l2_eps), _stream(v, stream))


@_typed
def gdn_recurrence_seq_ex(state, q, k, v, g, beta, y, scale, snaps=None,
                          variant=GDN_RECUR_EXACT, stream=None):
    """state [N][H][S][S] in place; q, k [N][T][HK][S]; v, y [N][T][H][S];
    g, beta [N][T][H]; snaps None or [N][T][H][S][S] (state after each token);
    variant GDN_RECUR_EXACT or GDN_RECUR_T4 (the read-out of gdn_recurrence_ex)."""
    N, T, H, S = v.shape
    HK = q.shape[2]
    _shape(state, (N, H, S, S), "state")
    _shape(q, (N, T, HK, S), "q")
    _shape(k, (N, T, HK, S), "k")
    _shape(y, (N, T, H, S), "y")
    _shape(g, (N, T, H), "g")
    _shape(beta, (N, T, H), "beta")
    sp = None
    if snaps is not None:
        _shape(snaps, (N, T, H, S, S), "snaps")
        sp = _ptr(snaps, F32, "snaps")
    _call("gdn_recurrence_seq_ex", _ptr(state, F32, "state"), _ptr(q, F32, "q"), _ptr(k, F32, "k"),
          _ptr(v, F32, "v"), _ptr(g, F32, "g"), _ptr(beta, F32, "beta"), _ptr(y, F32, "y"), sp,
          N, T, HK, H, S, float(scale), int(variant), _stream(v, stream))


@_typed
def gdn_conv1d_silu_seq_ex(x, w, conv_state, out, snaps=None, stream=None):
    """gdn_conv1d_silu_seq with snaps None or [N][T][C][K-1] (history after
    each position)."""
    N, T, C = x.shape
    K = w.shape[1]
    _shape(w, (C, K), "w")
    _shape(conv_state, (N, C, K - 1), "conv_state")
    _shape(out, (N, T, C), "out")
    sp = None
    if snaps is not None:
        _shape(snaps, (N, T, C, K - 1), "snaps")
        sp = _ptr(snaps, F32, "snaps")
    _call("gdn_conv1d_silu_seq_ex", _ptr(x, F32, "x"), _ptr(w, F32, "w"),
          _ptr(conv_state, F32, "conv_state"), _ptr(out, F32, "out"), sp, N, T, C, K,
          _stream(x, stream))


@_typed
def gdn_gated_rmsnorm(y, w, z, out, eps=1e-6, stream=None):
    """y, z, out [..., D]; w [D]."""
    D = w.shape[0]
    _shape(z, y.shape, "z")
    _shape(out, y.shape, "out")
    if y.shape[-1] != D:
        raise ValueError("last dim of y must equal len(w)")
    _call("gdn_gated_rmsnorm", _ptr(y, F32, "y"), _ptr(w, F32, "w"), _ptr(z, F32, "z"),
          _ptr(out, F32, "out"), y.numel() // max(D, 1), D, float(eps), _stream(y, stream))


@_typed
def gdn_decode_block_bf16(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out,
                          n_k_heads, scale, l2_eps=1e-6, eps=1e-6, stream=None):
    """One fused decode layer. qkv [N][C] and z [N][H][S] hold bf16 bit patterns
    (int16/uint16 tensors, or torch.bfloat16); the rest are fp32:
    a, b [N][H]; conv_w [C][K]; ssm_a, dt_bias [H]; norm_w [S];
    conv_state [N][C][K-1] and state [N][H][S][S] updated in place; out [N][H][S]."""
    N, H, S = z.shape
    C, K = conv_w.shape
    _block_shapes(qkv, a, b, ssm_a, dt_bias, norm_w, conv_state, state, out, N, H, S, C, K,
                  n_k_heads)
    _call("gdn_decode_block_bf16", _ptr16(qkv, "qkv"), _ptr16(z, "z"), _ptr(a, F32, "a"),
          _ptr(b, F32, "b"), _ptr(conv_w, F32, "conv_w"), _ptr(ssm_a, F32, "ssm_a"),
          _ptr(dt_bias, F32, "dt_bias"), _ptr(norm_w, F32, "norm_w"),
          _ptr(conv_state, F32, "conv_state"), _ptr(state, F32, "state"), _ptr(out, F32, "out"),
          N, n_k_heads, H, S, K, float(scale), float(l2_eps), float(eps), _stream(z, stream))


def gdn_decode_block_workspace_bytes(n_seqs, n_k_heads, n_v_heads) -> int:
    return int(load_library().gdn_decode_block_workspace_bytes(n_seqs, n_k_heads, n_v_heads))


@_typed
def gdn_decode_block_bf16_noalloc(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state,
                                  state, out, n_k_heads, scale, l2_eps=1e-6, eps=1e-6,
                                  stream=None):
    """gdn_decode_block_bf16_ex without a workspace: the counters live in the
    library's own per-GPU array (n_seqs * (HK + H) <= GDN_NOALLOC_MAX_COUNTERS);
    calls that overlap on one GPU race."""
    N, H, S = z.shape
    C, K = conv_w.shape
    _block_shapes(qkv, a, b, ssm_a, dt_bias, norm_w, conv_state, state, out, N, H, S, C, K,
                  n_k_heads)
    _call("gdn_decode_block_bf16_noalloc", _ptr16(qkv, "qkv"), _ptr16(z, "z"),
          _ptr(a, F32, "a"), _ptr(b, F32, "b"), _ptr(conv_w, F32, "conv_w"),
          _ptr(ssm_a, F32, "ssm_a"), _ptr(dt_bias, F32, "dt_bias"), _ptr(norm_w, F32, "norm_w"),
          _ptr(conv_state, F32, "conv_state"), _ptr(state, F32, "state"), _ptr(out, F32, "out"),
          N, n_k_heads, H, S, K, float(scale), float(l2_eps), float(eps), _stream(z, stream))


@_typed
def gdn_decode_block_bf16_ex(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state,
                             out, workspace, n_k_heads, scale, l2_eps=1e-6, eps=1e-6,
                             stream=None):
    """gdn_decode_block_bf16 with the state split over 64-row workgroups.
    Arguments as gdn_decode_block_bf16, plus workspace: a uint8 device tensor
    of at least gdn_decode_block_workspace_bytes(N, n_k_heads, H) bytes that
    is zero before the first call (every completed call leaves it zero)."""
    N, H, S = z.shape
    C, K = conv_w.shape
    _block_shapes(qkv, a, b, ssm_a, dt_bias, norm_w, conv_state, state, out, N, H, S, C, K,
                  n_k_heads)
    _call("gdn_decode_block_bf16_ex", _ptr16(qkv, "qkv"), _ptr16(z, "z"), _ptr(a, F32, "a"),
          _ptr(b, F32, "b"), _ptr(conv_w, F32, "conv_w"), _ptr(ssm_a, F32, "ssm_a"),
          _ptr(dt_bias, F32, "dt_bias"), _ptr(norm_w, F32, "norm_w"),
          _ptr(conv_state, F32, "conv_state"), _ptr(state, F32, "state"), _ptr(out, F32, "out"),
          _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
          N, n_k_heads, H, S, K, float(scale), float(l2_eps), float(eps), _stream(z, stream))


def _block_shapes(qkv, a, b, ssm_a, dt_bias, norm_w, conv_state, state, out, N, H, S, C, K,
                  n_k_heads):
    _shape(qkv, (N, C), "qkv")
    for t, nm in ((a, "a"), (b, "b")):
        _shape(t, (N, H), nm)
    _shape(ssm_a, (H,), "ssm_a")
    _shape(dt_bias, (H,), "dt_bias")
    _shape(norm_w, (S,), "norm_w")
    _shape(conv_state, (N, C, K - 1), "conv_state")
    _shape(state, (N, H, S, S), "state")
    _shape(out, (N, H, S), "out")
    if C != 2 * n_k_heads * S + H * S:
        raise ValueError(f"conv_dim {C} != 2*n_k_heads*S + n_v_heads*S")


def _ptr16(t: torch.Tensor, what: str) -> int:
    if t.dtype not in (torch.int16, torch.bfloat16) and t.dtype != getattr(torch, "uint16", None):
        raise TypeError(f"{what} must hold bf16 bit patterns (int16/uint16/bfloat16), got {t.dtype}")
    return _ptr(t, t.dtype, what)


def gdn_prefill_workspace_bytes(n_seqs, n_tokens, n_k_heads, n_v_heads, state_size) -> int:
    return int(load_library().gdn_prefill_workspace_bytes(n_seqs, n_tokens, n_k_heads, n_v_heads,
                                                          state_size))


@_typed
def gdn_prefill_bf16(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out,
                     workspace, n_k_heads, scale, l2_eps=1e-6, eps=1e-6, stream=None, scan=None):
    """One layer over T positions. qkv [N][T][C] and z [N][T][H][S] hold bf16
    bit patterns; a, b [N][T][H]; conv_w [C][K]; ssm_a, dt_bias [H]; norm_w [S];
    conv_state [N][C][K-1] and state [N][H][S][S] updated in place;
    out [N][T][H][S]; workspace a uint8 device tensor of at least
    gdn_prefill_workspace_bytes(...) bytes. scan=None calls gdn_prefill_bf16;
    GDN_SCAN_SEQUENTIAL or GDN_SCAN_CHUNKED call gdn_prefill_bf16_ex."""
    N, T, H, S = z.shape
    C, K = conv_w.shape
    _shape(qkv, (N, T, C), "qkv")
    for t, nm in ((a, "a"), (b, "b")):
        _shape(t, (N, T, H), nm)
    _shape(ssm_a, (H,), "ssm_a")
    _shape(dt_bias, (H,), "dt_bias")
    _shape(norm_w, (S,), "norm_w")
    _shape(conv_state, (N, C, K - 1), "conv_state")
    _shape(state, (N, H, S, S), "state")
    _shape(out, (N, T, H, S), "out")
    if C != 2 * n_k_heads * S + H * S:
        raise ValueError(f"conv_dim {C} != 2*n_k_heads*S + n_v_heads*S")
    args = (_ptr16(qkv, "qkv"), _ptr16(z, "z"), _ptr(a, F32, "a"),
            _ptr(b, F32, "b"), _ptr(conv_w, F32, "conv_w"), _ptr(ssm_a, F32, "ssm_a"),
            _ptr(dt_bias, F32, "dt_bias"), _ptr(norm_w, F32, "norm_w"),
            _ptr(conv_state, F32, "conv_state"), _ptr(state, F32, "state"), _ptr(out, F32, "out"),
            _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), N, T, n_k_heads, H, S, K,
            float(scale), float(l2_eps), float(eps))
    if scan is None:
        _call("gdn_prefill_bf16", *args, _stream(z, stream))
    else:
        _call("gdn_prefill_bf16_ex", *args, int(scan), _stream(z, stream))


def gdn_chunked_workspace_bytes(n_seqs, n_tokens, n_v_heads, state_size) -> int:
    return int(load_library().gdn_chunked_workspace_bytes(n_seqs, n_tokens, n_v_heads, state_size))


@_typed
def gdn_recurrence_seq_chunked(state, q, k, v, g, beta, y, scale, workspace, stream=None):
    """Chunked scan. state [N][H][S][S] in place; q, k [N][T][HK][S];
    v, y [N][T][H][S]; g, beta [N][T][H]; workspace a uint8 device tensor of
    at least gdn_chunked_workspace_bytes(N, T, H, S) bytes."""
    N, T, H, S = v.shape
    HK = q.shape[2]
    _shape(state, (N, H, S, S), "state")
    _shape(q, (N, T, HK, S), "q")
    _shape(k, (N, T, HK, S), "k")
    _shape(y, (N, T, H, S), "y")
    _shape(g, (N, T, H), "g")
    _shape(beta, (N, T, H), "beta")
    _call("gdn_recurrence_seq_chunked", _ptr(state, F32, "state"), _ptr(q, F32, "q"),
          _ptr(k, F32, "k"), _ptr(v, F32, "v"), _ptr(g, F32, "g"), _ptr(beta, F32, "beta"),
          _ptr(y, F32, "y"), _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
          N, T, HK, H, S, float(scale), _stream(v, stream))
