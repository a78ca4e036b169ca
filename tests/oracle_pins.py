"""Pins of the oracle: facts the pages and the mathematics fix, independent of it.

Each ``pin_*`` takes two bound oracle libraries (float and double builds) and
raises AssertionError when the oracle disagrees with the fact. The expected
values never come from the oracle itself: they are the hand-worked golden
examples, closed forms evaluated here in float64, special cases that reduce to
textbook formulas, invariants, or an independent float64 restatement (the
matrix form of the rule). ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on deliberately broken copies of it, each
of which must fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b)
    bad = err > atol + rtol * np.abs(b)
    assert not bad.any(), f"{what}: max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"


def _rand_case(rng, N=2, T=5, H=3, S=8, zero_state=False):
    """Random inputs of the recurrence with unit-norm k and q, g <= 0, beta in (0,1)."""
    q = _unit(rng, (N, T, H, S))
    k = _unit(rng, (N, T, H, S))
    v = rng.standard_normal((N, T, H, S))
    g = -np.abs(rng.standard_normal((N, T, H))) * 0.5
    beta = 1 / (1 + np.exp(-rng.standard_normal((N, T, H))))
    st = np.zeros((N, H, S, S)) if zero_state else rng.standard_normal((N, H, S, S)) * 0.3
    # everything exactly representable in fp32, so both builds see the same inputs
    f = lambda x: x.astype(np.float32).astype(np.float64)
    return f(st), f(q), f(k), f(v), f(g), f(beta)


# ---------------------------------------------------------------------------
# Recurrence
# ---------------------------------------------------------------------------

def pin_recurrence_golden(L32, L64):
    """Hand-worked S=2, T=3 example (all dyadic): exact in both builds."""
    e = _golden()["recurrence_s2"]
    st0 = np.array(e["state0_rows"])[None, None]          # [1][1][S][S] rows j
    q = np.array(e["q"])[None, :, None, :]
    k = np.array(e["k"])[None, :, None, :]
    v = np.array(e["v"])[None, :, None, :]
    g = np.array(e["g"])[None, :, None]
    b = np.array(e["beta"])[None, :, None]
    for L in (L32, L64):
        y, st = oracle.recurrence_seq(st0, q, k, v, g, b, e["scale"], prec=L)
        assert np.array_equal(y[0, :, 0, :], np.array(e["y"])), y[0, :, 0, :]
        assert np.array_equal(st[0, 0], np.array(e["state_final_rows"])), st[0, 0]


def pin_recurrence_beta0_decay_only(L32, L64):
    """beta = 0: the state only decays, M_T = (prod_t e^{g_t}) M_0, and
    y_t = scale * (decayed rows) . q_t."""
    rng = np.random.default_rng(11)
    st, q, k, v, g, _ = _rand_case(rng, N=2, T=6, H=2, S=16)
    beta = np.zeros_like(g)
    scale = 0.25
    cum = np.exp(np.cumsum(g, axis=1))                     # [N][T][H]
    y_ref = np.einsum("nhji,nthi->nthj", st, q) * cum[..., None] * scale
    st_ref = st * cum[:, -1][:, :, None, None]
    for L, tol in ((L64, 1e-12), (L32, 2e-6)):
        y, s = oracle.recurrence_seq(st, q, k, v, g, beta, scale, prec=L)
        _close(y, y_ref, tol, tol, "beta=0 y")
        _close(s, st_ref, tol, tol, "beta=0 state")


def pin_recurrence_projection(L32, L64):
    """g = 0, beta = 1, |k| = 1: after one step M k = v (the row's prediction
    of k is v_j exactly) and M u = M_prev u for every u orthogonal to k."""
    rng = np.random.default_rng(12)
    N, H, S = 1, 2, 16
    st, q, _, v, g, _ = _rand_case(rng, N=N, T=1, H=H, S=S)
    k = _unit(rng, (N, 1, H, S))      # exactly unit in float64 (not rounded to fp32)
    g = np.zeros_like(g)
    beta = np.ones_like(g)
    kk = k[:, 0]                                           # [N][H][S]
    u = rng.standard_normal((N, H, S))
    u -= np.sum(u * kk, -1, keepdims=True) * kk            # orthogonal to k
    for L, tol in ((L64, 1e-12), (L32, 1e-5)):
        _, s = oracle.recurrence_seq(st, q, k, v, g, beta, 1.0, prec=L)
        _close(np.einsum("nhji,nhi->nhj", s, kk), v[:, 0], tol, tol, "M k = v")
        _close(np.einsum("nhji,nhi->nhj", s, u), np.einsum("nhji,nhi->nhj", st, u),
               tol, tol, "M u = M_prev u")


def pin_recurrence_s1_closed_form(L32, L64):
    """S = 1 (k, q = +-1): s_t = (1 - b_t) e^{g_t} s_{t-1} + b_t k_t v_t and
    y_t = scale q_t s_t; unrolled, s_T = sum_t (prod_{tau>t} a_tau) c_t
    + (prod a) s_0 with a_t = (1 - b_t) e^{g_t}, c_t = b_t k_t v_t."""
    rng = np.random.default_rng(13)
    T = 40
    k = rng.choice([-1.0, 1.0], T)
    q = rng.choice([-1.0, 1.0], T)
    v = rng.standard_normal(T).astype(np.float32).astype(np.float64)
    g = (-np.abs(rng.standard_normal(T)) * 0.3).astype(np.float32).astype(np.float64)
    b = rng.uniform(0.05, 0.95, T).astype(np.float32).astype(np.float64)
    s0 = 0.75
    a = (1 - b) * np.exp(g)
    c = b * k * v
    s_ref = np.empty(T)
    for t in range(T):
        s_ref[t] = sum(np.prod(a[tau + 1:t + 1]) * c[tau] for tau in range(t + 1)) \
            + np.prod(a[:t + 1]) * s0
    scale = 0.5
    y_ref = scale * q * s_ref
    shp = lambda x: x.reshape(1, T, 1, 1)
    for L, tol in ((L64, 1e-12), (L32, 2e-6)):
        y, s = oracle.recurrence_seq(np.full((1, 1, 1, 1), s0), shp(q), shp(k), shp(v),
                                     g.reshape(1, T, 1), b.reshape(1, T, 1), scale, prec=L)
        _close(y.ravel(), y_ref, tol, tol, "S=1 y")
        _close(s.ravel(), s_ref[-1:], tol, tol, "S=1 state")


def matrix_form(st, q, k, v, g, beta, scale):
    """Independent float64 restatement of the rule in matrix form:
    M_t = e^{g_t} M_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    y_t = scale * M_t q_t, with M the D_v x D_k matrix whose row j is the
    stored row j."""
    N, T, H, S = q.shape
    M = st.astype(np.float64).copy()
    y = np.empty((N, T, H, S))
    I = np.eye(S)
    for n in range(N):
        for h in range(H):
            for t in range(T):
                kt = k[n, t, h]
                M[n, h] = np.exp(g[n, t, h]) * M[n, h] @ (I - beta[n, t, h] * np.outer(kt, kt)) \
                    + beta[n, t, h] * np.outer(v[n, t, h], kt)
                y[n, t, h] = scale * (M[n, h] @ q[n, t, h])
    return y, M


def pin_recurrence_matrix_form(L32, L64):
    """The row-wise oracle agrees with the float64 matrix form (non-symmetric
    initial state, so a transposed layout would fail)."""
    rng = np.random.default_rng(14)
    st, q, k, v, g, beta = _rand_case(rng, N=2, T=7, H=3, S=8)
    scale = 1 / math.sqrt(8)
    y_ref, st_ref = matrix_form(st, q, k, v, g, beta, scale)
    for L, rtol, atol in ((L64, 1e-11, 1e-12), (L32, 1e-5, 1e-6)):
        y, s = oracle.recurrence_seq(st, q, k, v, g, beta, scale, prec=L)
        _close(y, y_ref, rtol, atol, "matrix form y")
        _close(s, st_ref, rtol, atol, "matrix form state")


def pin_recurrence_linear_in_v(L32, L64):
    """From a zero state y is linear in v: y(v1 + v2) = y(v1) + y(v2) and
    y(c v) = c y(v)."""
    rng = np.random.default_rng(15)
    st, q, k, v1, g, beta = _rand_case(rng, N=1, T=6, H=2, S=8, zero_state=True)
    v2 = rng.standard_normal(v1.shape)
    f = lambda vv: oracle.recurrence_seq(st, q, k, vv, g, beta, 0.3, prec=L64)[0]
    _close(f(v1 + v2), f(v1) + f(v2), 1e-10, 1e-12, "additivity")
    _close(f(2.5 * v1), 2.5 * f(v1), 1e-10, 1e-12, "homogeneity")


def pin_recurrence_scan_equals_steps(L32, L64):
    """A scan over T tokens equals T chained single-token steps, bit for bit."""
    rng = np.random.default_rng(16)
    st, q, k, v, g, beta = _rand_case(rng, N=2, T=9, H=2, S=8)
    for L in (L32, L64):
        y, s = oracle.recurrence_seq(st, q, k, v, g, beta, 0.4, prec=L)
        s2 = st
        for t in range(q.shape[1]):
            yt, s2 = oracle.recurrence(s2, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], 0.4, prec=L)
            assert np.array_equal(yt, y[:, t]), f"token {t}"
        assert np.array_equal(s2, s)


def pin_recurrence_split_resume(L32, L64):
    """scan(T1) then scan(T2) from the saved state equals scan(T1 + T2)."""
    rng = np.random.default_rng(17)
    st, q, k, v, g, beta = _rand_case(rng, N=1, T=10, H=2, S=8)
    for L in (L32, L64):
        y, s = oracle.recurrence_seq(st, q, k, v, g, beta, 0.4, prec=L)
        ya, sa = oracle.recurrence_seq(st, q[:, :4], k[:, :4], v[:, :4], g[:, :4], beta[:, :4], 0.4, prec=L)
        yb, sb = oracle.recurrence_seq(sa, q[:, 4:], k[:, 4:], v[:, 4:], g[:, 4:], beta[:, 4:], 0.4, prec=L)
        assert np.array_equal(np.concatenate([ya, yb], axis=1), y)
        assert np.array_equal(sb, s)


def pin_recurrence_rows_independent(L32, L64):
    """Permuting the value rows j (state rows and v entries together) permutes
    y and the final state the same way."""
    rng = np.random.default_rng(18)
    st, q, k, v, g, beta = _rand_case(rng, N=1, T=5, H=2, S=8)
    perm = rng.permutation(8)
    y, s = oracle.recurrence_seq(st, q, k, v, g, beta, 0.4, prec=L32)
    yp, sp = oracle.recurrence_seq(st[:, :, perm], q, k, v[..., perm], g, beta, 0.4, prec=L32)
    assert np.array_equal(yp, y[..., perm])
    assert np.array_equal(sp, s[:, :, perm])


def pin_recurrence_bounded(L32, L64):
    """With |k| = 1, beta in (0,1) and decay <= 1 the homogeneous map has
    spectral norm <= 1, so ||M_t||_F <= ||M_{t-1}||_F + beta_t ||v_t||: checked
    step by step over 300 tokens, and the values stay finite."""
    rng = np.random.default_rng(19)
    st, q, k, v, g, beta = _rand_case(rng, N=1, T=300, H=1, S=16)
    s = st
    for t in range(q.shape[1]):
        _, s_new = oracle.recurrence(s, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], 0.25, prec=L32)
        bound = np.linalg.norm(s) + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.all(np.isfinite(s_new))
        assert np.linalg.norm(s_new) <= bound * (1 + 1e-5) + 1e-6, t
        s = s_new


def pin_recurrence_f32_vs_f64(L32, L64):
    """The float build stays within the parity tolerance of the double build on
    the tiny workload's shapes (S = 32, T = 8) and on a 512-token scan."""
    rng = np.random.default_rng(20)
    for T, rtol in ((8, 1e-5), (512, 1e-4)):
        st, q, k, v, g, beta = _rand_case(rng, N=1, T=T, H=2, S=32)
        y32, s32 = oracle.recurrence_seq(st, q, k, v, g, beta, 1 / math.sqrt(32), prec=L32)
        y64, s64 = oracle.recurrence_seq(st, q, k, v, g, beta, 1 / math.sqrt(32), prec=L64)
        _close(y32, y64, rtol, 1e-6, f"f32 vs f64 y T={T}")
        _close(s32, s64, rtol, 1e-6, f"f32 vs f64 state T={T}")


# ---------------------------------------------------------------------------
# Conv1d + SiLU
# ---------------------------------------------------------------------------

def _silu64(x):
    return x / (1 + np.exp(-x))


def pin_conv_golden(L32, L64):
    e = _golden()["conv_k4"]
    w = np.array(e["w"])[None]
    cs0 = np.array(e["history0"])[None, None]
    x = np.array(e["x"]).reshape(1, 2, 1)
    pre = np.array(e["pre_activation"])
    for L in (L32, L64):
        out, cs = oracle.conv1d_silu_seq(x, w, cs0, prec=L)
        _close(out.ravel(), _silu64(pre), 3e-7, 0, "conv golden out")
        assert np.array_equal(cs.ravel(), np.array(e["history_final"]))


def pin_conv_impulse(L32, L64):
    """Zero history, a unit impulse at step 0: out at step tau is
    silu(w[c][K-1-tau]) for tau < K, then silu(0) = 0."""
    rng = np.random.default_rng(21)
    C, K, T = 5, 4, 7
    w = rng.standard_normal((C, K)).astype(np.float32)
    x = np.zeros((1, T, C))
    x[0, 0, :] = 1.0
    for L in (L32, L64):
        out, _ = oracle.conv1d_silu_seq(x, w, np.zeros((1, C, K - 1)), prec=L)
        ref = np.zeros((T, C))
        for tau in range(K):
            ref[tau] = _silu64(w[:, K - 1 - tau].astype(np.float64))
        _close(out[0], ref, 3e-7, 0, "impulse response")


def pin_conv_history_is_last_inputs(L32, L64):
    """After T >= K-1 steps the history holds the last K-1 raw inputs."""
    rng = np.random.default_rng(22)
    N, T, C, K = 2, 6, 9, 4
    x = rng.standard_normal((N, T, C)).astype(np.float32)
    w = rng.standard_normal((C, K))
    cs0 = rng.standard_normal((N, C, K - 1))
    for L in (L32, L64):
        _, cs = oracle.conv1d_silu_seq(x, w, cs0, prec=L)
        assert np.array_equal(cs, np.transpose(x[:, T - (K - 1):, :], (0, 2, 1)).astype(cs.dtype))


def pin_conv_scan_equals_steps(L32, L64):
    rng = np.random.default_rng(23)
    N, T, C, K = 2, 5, 7, 3
    x = rng.standard_normal((N, T, C))
    w = rng.standard_normal((C, K))
    cs0 = rng.standard_normal((N, C, K - 1))
    for L in (L32, L64):
        out, cs = oracle.conv1d_silu_seq(x, w, cs0, prec=L)
        c2 = cs0
        for t in range(T):
            o, c2 = oracle.conv1d_silu(x[:, t], w, c2, prec=L)
            assert np.array_equal(o, out[:, t])
        assert np.array_equal(c2, cs)


def pin_conv_direct_correlation(L32, L64):
    """Against a float64 causal correlation over the history-padded signal:
    out[t][c] = silu(sum_u w[c][u] * xp[t + u][c]), xp = history ++ x."""
    rng = np.random.default_rng(24)
    N, T, C, K = 2, 11, 6, 4
    x = rng.standard_normal((N, T, C)).astype(np.float32).astype(np.float64)
    w = rng.standard_normal((C, K)).astype(np.float32).astype(np.float64)
    cs0 = rng.standard_normal((N, C, K - 1)).astype(np.float32).astype(np.float64)
    xp = np.concatenate([np.transpose(cs0, (0, 2, 1)), x], axis=1)   # [N][K-1+T][C]
    pre = np.zeros((N, T, C))
    for u in range(K):
        pre += w[:, u][None, None, :] * xp[:, u:u + T, :]
    for L, tol in ((L64, 1e-12), (L32, 2e-6)):
        out, _ = oracle.conv1d_silu_seq(x, w, cs0, prec=L)
        _close(out, _silu64(pre), tol, tol, "direct correlation")


# ---------------------------------------------------------------------------
# Gated RMSNorm
# ---------------------------------------------------------------------------

def pin_norm_golden(L32, L64):
    e = _golden()["gated_norm_d4"]
    for L in (L32, L64):
        out = oracle.gated_rmsnorm(e["y"], e["w"], e["z"], eps=e["eps"], prec=L)
        _close(out, np.array(e["out"]), 4e-7, 0, "norm golden")


def pin_norm_mean_square(L32, L64):
    """With w = 1: mean((out / silu(z))^2) = s / (s + D eps), s = sum y^2 / ...
    i.e. mean(y^2) / (mean(y^2) + eps), with eps comparable to mean(y^2)."""
    rng = np.random.default_rng(25)
    D, R = 16, 5
    f = lambda x: x.astype(np.float32).astype(np.float64)
    y = f(rng.standard_normal((R, D)) * 0.1)
    z = f(rng.uniform(1, 3, (R, D)))
    eps = 0.01
    ms = np.mean(y ** 2, axis=1)
    for L, tol in ((L64, 1e-12), (L32, 2e-6)):
        out = oracle.gated_rmsnorm(y, np.ones(D), z, eps=eps, prec=L)
        r = out / _silu64(z)
        _close(np.mean(r ** 2, axis=1), ms / (ms + eps), tol, tol, "mean square")


def pin_norm_direct(L32, L64):
    rng = np.random.default_rng(26)
    R, D = 7, 32
    y, z = rng.standard_normal((R, D)), rng.standard_normal((R, D))
    w = 1 + 0.1 * rng.standard_normal(D)
    f = lambda x: x.astype(np.float32).astype(np.float64)
    y, z, w = f(y), f(z), f(w)
    ref = y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + 1e-6) * w * _silu64(z)
    for L, tol in ((L64, 1e-12), (L32, 2e-6)):
        _close(oracle.gated_rmsnorm(y, w, z, eps=1e-6, prec=L), ref, tol, tol, "norm direct")


def pin_norm_scale_invariant(L32, L64):
    rng = np.random.default_rng(27)
    y, z = rng.standard_normal((3, 16)), rng.standard_normal((3, 16))
    w = rng.standard_normal(16)
    a = oracle.gated_rmsnorm(y, w, z, eps=1e-9, prec=L64)
    b = oracle.gated_rmsnorm(8.0 * y, w, z, eps=1e-9, prec=L64)
    _close(a, b, 1e-8, 1e-10, "scale invariance")


# ---------------------------------------------------------------------------
# Decay gate and sigmoid
# ---------------------------------------------------------------------------

def pin_gate_zero_preactivation(L32, L64):
    """u = 0: softplus(0) = ln 2, so g = -exp(A_log) ln 2."""
    A_log = np.array([-1.0, 0.0, 0.5, 2.0])
    for L, tol in ((L64, 1e-15), (L32, 3e-7)):
        g = oracle.decay_gate(np.zeros((1, 4)), np.zeros(4), A_log, prec=L)
        _close(g[0], -np.exp(A_log) * math.log(2), tol, 0, "g at u=0")


def pin_gate_reference(L32, L64):
    """Against float64 math.log1p(math.exp(u)) with a non-zero dt_bias, and a
    finite g for very large pre-activations."""
    rng = np.random.default_rng(28)
    H = 6
    a = rng.standard_normal((50, H)) * 8
    a[0] = [25.0, 1e4, 1e30, -80.0, 19.5, 20.5]
    dt = (rng.standard_normal(H) * 0.5).astype(np.float32).astype(np.float64)
    A_log = rng.standard_normal(H)
    f = lambda x: x.astype(np.float32).astype(np.float64)
    a32, A32 = f(a), f(A_log)
    for L, tol in ((L64, 1e-13), (L32, 5e-6)):
        g = oracle.decay_gate(a32, dt, A32, prec=L)
        assert np.all(np.isfinite(g)) and np.all(g <= 0)
        u = (a32 + dt[None, :])
        if L is L32:
            u = f(u)
        sp = np.array([[ui if ui > 20 else math.log1p(math.exp(ui)) for ui in row] for row in u])
        _close(g, -np.exp(A32)[None, :] * sp, tol, 1e-30, "gate vs log1p(exp)")


def pin_gate_continuous_at_guard(L32, L64):
    """Across u = 20 the guarded softplus is continuous to well under an fp32
    ulp of 20 (log1p(e^20) - 20 is about 2e-9)."""
    A_log = np.zeros(1)
    us = np.array([[20.0 - 1e-5], [20.0], [20.0 + 1e-5]])
    for L in (L32, L64):
        g = oracle.decay_gate(us, np.zeros(1), A_log, prec=L).ravel()
        assert abs(g[1] - g[0]) < 2e-5 and abs(g[2] - g[1]) < 2e-5, g
        assert abs(g[1] + 20.0) < 4e-6


def pin_sigmoid(L32, L64):
    x = np.array([-30.0, -3.0, -0.5, 0.0, 0.5, 3.0, 30.0])
    for L, tol in ((L64, 1e-15), (L32, 3e-7)):
        s = oracle.sigmoid(x, prec=L)
        _close(s, 1 / (1 + np.exp(-x)), tol, 1e-30, "sigmoid")
        _close(oracle.sigmoid(-x, prec=L) + s, np.ones_like(x), tol, tol, "sigmoid symmetry")


# ---------------------------------------------------------------------------
# L2 normalisation and grouped-query repeat
# ---------------------------------------------------------------------------

def pin_l2norm_unit_and_tiled_repeat(L32, L64):
    rng = np.random.default_rng(29)
    rows, HK, H, S = 3, 4, 8, 16
    x = rng.standard_normal((rows, HK, S))
    for L, tol in ((L64, 1e-14), (L32, 1e-6)):
        out = oracle.l2norm_gqa(x, H, eps=1e-6, prec=L)
        _close(np.linalg.norm(out, axis=-1), np.ones((rows, H)), tol, 0, "unit norm")
        for vh in range(H):
            assert np.array_equal(out[:, vh], out[:, vh % HK]), vh
        _close(out[:, :HK], x / np.linalg.norm(x, axis=-1, keepdims=True), tol, tol, "direction")


def pin_l2norm_eps_floor(L32, L64):
    """A vector shorter than eps is divided by eps, not by its length."""
    x = np.zeros((1, 2, 4))
    x[0, 0] = [1e-9, -2e-9, 0.0, 3e-9]
    for L in (L32, L64):
        out = oracle.l2norm_gqa(x, 2, eps=1e-6, prec=L)
        _close(out[0, 0], x[0, 0] / 1e-6, 1e-6, 0, "eps floor")
        assert np.all(out[0, 1] == 0)


# ---------------------------------------------------------------------------
# Decode block
# ---------------------------------------------------------------------------

def pin_block_is_composition(L32, L64):
    """The one-layer block equals the stages chained by hand (bitwise), with
    the split [q | k | v] of the conv output and the tiled repeat."""
    from linear_attention_ssm_recurrence_amd import inputs
    rng = np.random.default_rng(30)
    N, HK, H, S, K = 2, 2, 4, 8, 4
    C = 2 * HK * S + H * S
    bits = lambda x: inputs.to_bf16_bits(x.astype(np.float32))
    qkv = bits(rng.standard_normal((N, C)))
    z = bits(rng.standard_normal((N, H, S)))
    a, b = rng.standard_normal((N, H)), rng.standard_normal((N, H))
    cw = rng.standard_normal((C, K)) * 0.5
    A_log, dt = rng.standard_normal(H), rng.standard_normal(H) * 0.1
    nw = 1 + 0.1 * rng.standard_normal(S)
    cs0 = rng.standard_normal((N, C, K - 1))
    st0 = rng.standard_normal((N, H, S, S)) * 0.05
    scale = 1 / math.sqrt(S)
    for L in (L32, L64):
        out, cs, st = oracle.decode_block_bf16(qkv, z, a, b, cw, A_log, dt, nw, cs0, st0,
                                               HK, scale, 1e-6, 1e-6, prec=L)
        x = inputs.bf16_bits_to_f32(qkv)
        co, cs_ref = oracle.conv1d_silu(x, cw, cs0, prec=L)
        qn = oracle.l2norm_gqa(co[:, :HK * S].reshape(N, HK, S), H, 1e-6, prec=L)
        kn = oracle.l2norm_gqa(co[:, HK * S:2 * HK * S].reshape(N, HK, S), H, 1e-6, prec=L)
        vv = co[:, 2 * HK * S:].reshape(N, H, S)
        bt = oracle.sigmoid(b, prec=L)
        gt = oracle.decay_gate(a, dt, A_log, prec=L)
        y, st_ref = oracle.recurrence(st0, qn, kn, vv, gt, bt, scale, prec=L)
        o_ref = oracle.gated_rmsnorm(y, nw, inputs.bf16_bits_to_f32(z), 1e-6, prec=L)
        assert np.array_equal(out, o_ref)
        assert np.array_equal(cs, cs_ref)
        assert np.array_equal(st, st_ref)


def _prefill_case(rng, N=2, T=6, HK=2, H=4, S=8, K=4):
    from linear_attention_ssm_recurrence_amd import inputs
    C = 2 * HK * S + H * S
    bits = lambda x: inputs.to_bf16_bits(x.astype(np.float32))
    return dict(qkv=bits(rng.standard_normal((N, T, C))), z=bits(rng.standard_normal((N, T, H, S))),
                a=rng.standard_normal((N, T, H)), b=rng.standard_normal((N, T, H)),
                conv_w=rng.standard_normal((C, K)) * 0.5, A_log=rng.standard_normal(H),
                dt_bias=rng.standard_normal(H) * 0.1, norm_w=1 + 0.1 * rng.standard_normal(S),
                conv_state=rng.standard_normal((N, C, K - 1)),
                state=rng.standard_normal((N, H, S, S)) * 0.05, HK=HK, scale=1 / math.sqrt(S))


def pin_prefill_is_chained_decode_layers(L32, L64):
    """The prefill over T positions equals T single-position decode layers
    chained (bitwise), so it composes the pinned stages the same way."""
    rng = np.random.default_rng(31)
    c = _prefill_case(rng)
    for L in (L32, L64):
        out, cs, st = oracle.prefill_bf16(c["qkv"], c["z"], c["a"], c["b"], c["conv_w"], c["A_log"],
                                          c["dt_bias"], c["norm_w"], c["conv_state"], c["state"],
                                          c["HK"], c["scale"], prec=L)
        cs2, st2 = c["conv_state"], c["state"]
        T = c["qkv"].shape[1]
        for t in range(T):
            o, cs2, st2 = oracle.decode_block_bf16(
                c["qkv"][:, t], c["z"][:, t], c["a"][:, t], c["b"][:, t], c["conv_w"], c["A_log"],
                c["dt_bias"], c["norm_w"], cs2, st2, c["HK"], c["scale"], prec=L)
            assert np.array_equal(o, out[:, t]), f"position {t}"
        assert np.array_equal(cs2, cs) and np.array_equal(st2, st)


ALL_PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
