"""Gated DeltaNet oracle: ctypes front end over the plain C implementation.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library and
its Python binding never import it.

Every function takes and returns NumPy arrays and copies its inputs, so the
caller's arrays are never modified; stateful steps return the updated state.
``prec`` selects the build: ``"f32"`` (the pages' precision, the parity
reference) or ``"f64"`` (the same steps in double precision, used to bound the
float build's own rounding).

Which page and section each step follows is stated beside each C function in
``gdn_oracle.c``. Parity is unpinned only where glibc's ``expf``/``log1pf``
and the device library round differently, and where reduction order differs;
both are covered by the tolerance, not by a pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIBS = {"f32": os.path.join(_HERE, "liboracle_f32.so"),
         "f64": os.path.join(_HERE, "liboracle_f64.so")}
_DTYPES = {"f32": np.float32, "f64": np.float64}

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fopenmp"]


def build(verbose: bool = False) -> None:
    """Compile the float and double builds of the oracle with gcc."""
    for prec, out in _LIBS.items():
        defs = ["-DORACLE_F64"] if prec == "f64" else []
        cmd = ["gcc", *CFLAGS, *defs, _SRC, "-o", out + ".tmp", "-lm"]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    _loaded.clear()


_loaded: dict = {}


def bind(path: str, prec: str):
    """Load an oracle shared library from ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    real = ctypes.c_double if prec == "f64" else ctypes.c_float
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    lib.oracle_precision.restype = ctypes.c_char_p
    lib.oracle_set_threads.argtypes = [I]
    lib.oracle_get_threads.restype = I
    lib.oracle_decay_gate.argtypes = [P, P, P, P, I, L]
    lib.oracle_sigmoid.argtypes = [P, P, L]
    lib.oracle_l2norm_gqa.argtypes = [P, P, L, I, I, I, real]
    lib.oracle_conv1d_silu_seq.argtypes = [P, P, P, P, I, I, I, I]
    lib.oracle_recurrence_seq.argtypes = [P, P, P, P, P, P, P, I, I, I, I, real]
    lib.oracle_gated_rmsnorm.argtypes = [P, P, P, P, L, I, real]
    lib.oracle_decode_block_bf16.argtypes = [P] * 11 + [I] * 5 + [real] * 3
    lib.oracle_prefill_bf16.argtypes = [P] * 11 + [I] * 6 + [real] * 3
    for name in ("oracle_decay_gate", "oracle_sigmoid", "oracle_l2norm_gqa",
                 "oracle_conv1d_silu_seq", "oracle_recurrence_seq",
                 "oracle_gated_rmsnorm", "oracle_decode_block_bf16",
                 "oracle_prefill_bf16", "oracle_set_threads"):
        getattr(lib, name).restype = None
    if lib.oracle_precision().decode() != prec:
        raise RuntimeError(f"{path} is not the {prec} build")
    return lib


def _lib(prec: str):
    if not isinstance(prec, str):
        return prec          # an already-bound library (mutation tests)
    if prec not in _LIBS:
        raise ValueError(f"prec must be 'f32' or 'f64', got {prec!r}")
    lib = _loaded.get(prec)
    if lib is not None:
        return lib
    path = _LIBS[prec]
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        build()
    lib = bind(path, prec)
    _loaded[prec] = lib
    return lib


def _dtype(prec):
    if isinstance(prec, str):
        return _DTYPES[prec]
    return np.float64 if prec.oracle_precision().decode() == "f64" else np.float32


def _arr(x, prec):
    return np.ascontiguousarray(np.array(x, dtype=_dtype(prec), copy=True))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int, prec: str = "f32") -> None:
    _lib(prec).oracle_set_threads(int(n))


def get_threads(prec: str = "f32") -> int:
    return int(_lib(prec).oracle_get_threads())


def decay_gate(a, dt_bias, A_log, prec="f32"):
    """g[..., h] = -exp(A_log[h]) * softplus(a[..., h] + dt_bias[h])."""
    a = _arr(a, prec)
    dt_bias = _arr(dt_bias, prec)
    A_log = _arr(A_log, prec)
    H = A_log.shape[0]
    assert dt_bias.shape == (H,) and a.shape[-1] == H
    g = np.empty_like(a)
    _lib(prec).oracle_decay_gate(_p(a), _p(dt_bias), _p(A_log), _p(g), H, a.size // H)
    return g


def sigmoid(x, prec="f32"):
    x = _arr(x, prec)
    y = np.empty_like(x)
    _lib(prec).oracle_sigmoid(_p(x), _p(y), x.size)
    return y


def l2norm_gqa(x, n_v_heads, eps=1e-6, prec="f32"):
    """x [..., HK, S] -> [..., H, S]; V-head vh reads K-head vh mod HK."""
    x = _arr(x, prec)
    HK, S = x.shape[-2:]
    rows = x.size // (HK * S)
    out = np.empty(x.shape[:-2] + (n_v_heads, S), dtype=_dtype(prec))
    _lib(prec).oracle_l2norm_gqa(_p(x), _p(out), rows, HK, n_v_heads, S, eps)
    return out


def conv1d_silu_seq(x, w, conv_state, prec="f32"):
    """x [N][T][C], w [C][K], conv_state [N][C][K-1] -> (out, new_conv_state)."""
    x = _arr(x, prec)
    w = _arr(w, prec)
    cs = _arr(conv_state, prec)
    N, T, C = x.shape
    K = w.shape[1]
    assert w.shape == (C, K) and cs.shape == (N, C, K - 1)
    assert 1 <= K <= 65, "conv_kernel must be 1..65 (the oracle's history holds 64 taps)"
    out = np.empty_like(x)
    _lib(prec).oracle_conv1d_silu_seq(_p(x), _p(w), _p(cs), _p(out), N, T, C, K)
    return out, cs


def conv1d_silu(x, w, conv_state, prec="f32"):
    """One decode step: x [N][C] -> (out [N][C], new_conv_state)."""
    x = np.asarray(x)
    out, cs = conv1d_silu_seq(x[:, None, :], w, conv_state, prec)
    return out[:, 0, :], cs


def recurrence_seq(state, q, k, v, g, beta, scale, prec="f32"):
    """state [N][H][S][S]; q,k,v [N][T][H][S]; g,beta [N][T][H] -> (y, state)."""
    st = _arr(state, prec)
    q, k, v = (_arr(t, prec) for t in (q, k, v))
    g, beta = _arr(g, prec), _arr(beta, prec)
    N, T, H, S = q.shape
    assert st.shape == (N, H, S, S)
    assert k.shape == q.shape and v.shape == q.shape
    assert g.shape == (N, T, H) and beta.shape == (N, T, H)
    y = np.empty_like(q)
    _lib(prec).oracle_recurrence_seq(_p(st), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                     _p(y), N, T, H, S, float(scale))
    return y, st


def recurrence(state, q, k, v, g, beta, scale, prec="f32"):
    """One decode step: q,k,v [N][H][S]; g,beta [N][H] -> (y [N][H][S], state)."""
    q, k, v = (np.asarray(t)[:, None] for t in (q, k, v))
    g, beta = np.asarray(g)[:, None], np.asarray(beta)[:, None]
    y, st = recurrence_seq(state, q, k, v, g, beta, scale, prec)
    return y[:, 0], st


def gated_rmsnorm(y, w, z, eps=1e-6, prec="f32"):
    """y, z [..., D], w [D] -> out [..., D]."""
    y, w, z = _arr(y, prec), _arr(w, prec), _arr(z, prec)
    D = w.shape[0]
    assert y.shape == z.shape and y.shape[-1] == D
    out = np.empty_like(y)
    _lib(prec).oracle_gated_rmsnorm(_p(y), _p(w), _p(z), _p(out), y.size // D, D, eps)
    return out


def decode_block_bf16(qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state,
                      state, n_k_heads, scale, l2_eps=1e-6, eps=1e-6, prec="f32"):
    """One decode layer with bf16 activations (given as uint16 bit patterns).

    qkv [N][C] u16, z [N][H][S] u16, a, b [N][H], conv_w [C][K], A_log,
    dt_bias [H], norm_w [S], conv_state [N][C][K-1], state [N][H][S][S]
    -> (out [N][H][S], new_conv_state, new_state)
    """
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    z = np.ascontiguousarray(z, dtype=np.uint16)
    a, b = _arr(a, prec), _arr(b, prec)
    conv_w, A_log, dt_bias, norm_w = (_arr(t, prec) for t in (conv_w, A_log, dt_bias, norm_w))
    cs, st = _arr(conv_state, prec), _arr(state, prec)
    N, H, S = z.shape
    C, K = conv_w.shape
    assert qkv.shape == (N, C) and C == 2 * n_k_heads * S + H * S
    assert cs.shape == (N, C, K - 1) and st.shape == (N, H, S, S)
    out = np.empty((N, H, S), dtype=_dtype(prec))
    _lib(prec).oracle_decode_block_bf16(
        _p(qkv), _p(z), _p(a), _p(b), _p(conv_w), _p(A_log), _p(dt_bias), _p(norm_w),
        _p(cs), _p(st), _p(out), N, n_k_heads, H, S, K,
        float(scale), float(l2_eps), float(eps))
    return out, cs, st


def prefill_bf16(qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state, state, n_k_heads,
                 scale, l2_eps=1e-6, eps=1e-6, prec="f32"):
    """One layer over T positions with bf16 activations (uint16 bit patterns).

    qkv [N][T][C] u16, z [N][T][H][S] u16, a, b [N][T][H], conv_w [C][K],
    A_log, dt_bias [H], norm_w [S], conv_state [N][C][K-1], state [N][H][S][S]
    -> (out [N][T][H][S], new_conv_state, new_state)
    """
    qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
    z = np.ascontiguousarray(z, dtype=np.uint16)
    a, b = _arr(a, prec), _arr(b, prec)
    conv_w, A_log, dt_bias, norm_w = (_arr(t, prec) for t in (conv_w, A_log, dt_bias, norm_w))
    cs, st = _arr(conv_state, prec), _arr(state, prec)
    N, T, H, S = z.shape
    C, K = conv_w.shape
    assert qkv.shape == (N, T, C) and C == 2 * n_k_heads * S + H * S
    assert cs.shape == (N, C, K - 1) and st.shape == (N, H, S, S)
    out = np.empty((N, T, H, S), dtype=_dtype(prec))
    _lib(prec).oracle_prefill_bf16(
        _p(qkv), _p(z), _p(a), _p(b), _p(conv_w), _p(A_log), _p(dt_bias), _p(norm_w),
        _p(cs), _p(st), _p(out), N, T, n_k_heads, H, S, K,
        float(scale), float(l2_eps), float(eps))
    return out, cs, st
