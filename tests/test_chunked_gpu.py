"""Parity of the chunked scan (gdn_recurrence_seq_chunked) with the oracle's
sequential scan, within the fp32 tolerance (needs an MI355X)."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (DEV, RTOL_LONG_SCAN, assert_close, dev, host, oracle_threads,
                         prep_recurrence)
from linear_attention_ssm_recurrence_amd import gdn, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()
    oracle_threads()


def _case(rng, N, T, HK, H, S=128, state_sigma=0.05, a_log_shift=0.0):
    qh = oracle.l2norm_gqa(rng.standard_normal((N, T, HK, S)), HK)
    kh = oracle.l2norm_gqa(rng.standard_normal((N, T, HK, S)), HK)
    rep = lambda x: np.ascontiguousarray(x[:, :, np.arange(H) % HK, :])
    v = rng.standard_normal((N, T, H, S)).astype(np.float32)
    g = oracle.decay_gate(rng.standard_normal((N, T, H)), np.zeros(H),
                          rng.standard_normal(H) + a_log_shift)
    beta = oracle.sigmoid(rng.standard_normal((N, T, H)))
    st = (rng.standard_normal((N, H, S, S)) * state_sigma).astype(np.float32)
    return dict(qh=qh, kh=kh, q=rep(qh), k=rep(kh), v=v, g=g, beta=beta, state=st)


def _gpu_chunked(p, scale):
    N, T, H, S = p["v"].shape
    st = dev(p["state"])
    y = torch.empty((N, T, H, S), device=DEV)
    ws = torch.empty(gdn.gdn_chunked_workspace_bytes(N, T, H, S), dtype=torch.uint8, device=DEV)
    gdn.gdn_recurrence_seq_chunked(st, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                                   dev(p["beta"]), y, scale, ws)
    return y, st


@pytest.mark.parametrize("N,T,HK,H", [(1, 1, 2, 2), (1, 63, 2, 2), (1, 64, 2, 2),
                                       (2, 65, 2, 4), (1, 200, 1, 2), (3, 130, 4, 8)])
def test_chunked_vs_oracle(N, T, HK, H):
    rng = np.random.default_rng(800 + T + N)
    p = _case(rng, N, T, HK, H)
    scale = 1 / math.sqrt(128)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"], scale)
    y, st = _gpu_chunked(p, scale)
    assert_close(host(y), y_ref, f"chunked y N={N} T={T}")
    assert_close(host(st), st_ref, f"chunked state N={N} T={T}")


def test_chunked_strong_decay():
    """Heads whose decay underflows within a chunk (A_log shifted up by 4)."""
    rng = np.random.default_rng(77)
    p = _case(rng, 1, 150, 2, 4, a_log_shift=4.0)
    assert p["g"].min() < -50
    scale = 1 / math.sqrt(128)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"], scale)
    y, st = _gpu_chunked(p, scale)
    assert_close(host(y), y_ref, "chunked y, strong decay")
    assert_close(host(st), st_ref, "chunked state, strong decay")


def test_chunked_scan_4096():
    """1 sequence x 4096 tokens x 32 heads x S = 128, zero initial state."""
    w = inputs.WORKLOADS[3]
    d = inputs.draw(w, with_conv=False)
    p = prep_recurrence(d, w)
    p["qh"], p["kh"] = p["q"], p["k"]          # HK = H for this workload
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"], w.scale)
    y, st = _gpu_chunked(p, w.scale)
    assert_close(host(y), y_ref, "chunked y T=4096", rtol=RTOL_LONG_SCAN)
    assert_close(host(st), st_ref, "chunked state T=4096", rtol=RTOL_LONG_SCAN)


def _slice(p, a, b):
    """Positions a..b-1 of a case (the state is the case's initial state)."""
    out = {key: np.ascontiguousarray(val[:, a:b]) for key, val in p.items() if key != "state"}
    out["state"] = p["state"]
    return out


def test_chunked_split_resume():
    """Two chunked calls (T1 then T2, both splits inside a chunk) carry the
    state exactly like one sequential pass over T1 + T2 (oracle)."""
    rng = np.random.default_rng(901)
    N, T1, T2, HK, H = 2, 100, 91, 2, 4
    p = _case(rng, N, T1 + T2, HK, H)
    scale = 1 / math.sqrt(128)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"],
                                          scale)
    y1, st1 = _gpu_chunked(_slice(p, 0, T1), scale)
    p2 = _slice(p, T1, T1 + T2)
    p2["state"] = host(st1)
    y2, st2 = _gpu_chunked(p2, scale)
    assert_close(np.concatenate([host(y1), host(y2)], axis=1), y_ref, "chunked split/resume y")
    assert_close(host(st2), st_ref, "chunked split/resume state")


def test_chunked_many_blocks_gqa():
    """6 sequences x 300 positions, 8 -> 32 heads: 1536 scan blocks (several
    per CU, XCD grouping over many heads), ragged last chunk."""
    rng = np.random.default_rng(902)
    N, T, HK, H = 6, 300, 8, 32
    p = _case(rng, N, T, HK, H)
    scale = 1 / math.sqrt(128)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"],
                                          scale)
    y, st = _gpu_chunked(p, scale)
    assert_close(host(y), y_ref, "chunked 6x300 y")
    assert_close(host(st), st_ref, "chunked 6x300 state")


def test_chunked_vs_sequential_gpu_prefill_shape():
    """The prefill's shape (1 x 4096, 16 -> 32 heads, nonzero start state):
    the chunked scan against the sequential GPU scan on every head, and
    against the oracle on two sampled heads, within the long-scan tolerance."""
    rng = np.random.default_rng(903)
    N, T, HK, H = 1, 4096, 16, 32
    p = _case(rng, N, T, HK, H)
    scale = 1 / math.sqrt(128)
    y_c, st_c = _gpu_chunked(p, scale)
    st_s = dev(p["state"])
    y_s = torch.empty_like(y_c)
    gdn.gdn_recurrence_seq_ex(st_s, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                              dev(p["beta"]), y_s, scale)
    assert_close(host(y_c), host(y_s), "chunked vs sequential y", rtol=RTOL_LONG_SCAN)
    assert_close(host(st_c), host(st_s), "chunked vs sequential state", rtol=RTOL_LONG_SCAN)
    heads = [0, 31]                       # K-heads 0 and 15
    sub = lambda x: np.ascontiguousarray(x[:, :, heads])
    y_ref, st_ref = oracle.recurrence_seq(np.ascontiguousarray(p["state"][:, heads]), sub(p["q"]),
                                          sub(p["k"]), sub(p["v"]), sub(p["g"]), sub(p["beta"]),
                                          scale)
    assert_close(host(y_c)[:, :, heads], y_ref, "chunked y, sampled heads", rtol=RTOL_LONG_SCAN)
    assert_close(host(st_c)[:, heads], st_ref, "chunked state, sampled heads", rtol=RTOL_LONG_SCAN)


def test_chunked_infinite_decay():
    """g = -inf (the gate's output when exp(A_log) overflows) at the first, a
    middle and the last position of chunks: the decay exp(g) is 0 there, so
    the state restarts from k v^T terms alone, as in the oracle's sequential
    scan. Strongly negative finite g around it as well."""
    rng = np.random.default_rng(904)
    N, T, HK, H = 2, 200, 2, 4
    p = _case(rng, N, T, HK, H)
    g = p["g"].copy()
    g[0, 0, 0] = -np.inf          # first position of the sequence
    g[0, 37, 1] = -np.inf         # inside a chunk
    g[1, 63, 2] = -np.inf         # last position of a chunk
    g[1, 64, 3] = -np.inf         # first position of the next chunk
    g[0, 150:160, 2] = -1e30      # finite but far past underflow
    g[1, 199, 0] = -np.inf        # last position of the sequence
    p["g"] = g
    scale = 1 / math.sqrt(128)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"],
                                          scale)
    assert np.isfinite(y_ref).all() and np.isfinite(st_ref).all()
    y, st = _gpu_chunked(p, scale)
    assert_close(host(y), y_ref, "chunked y, infinite decay")
    assert_close(host(st), st_ref, "chunked state, infinite decay")
    st_s = dev(p["state"])
    y_s = torch.empty_like(y)
    gdn.gdn_recurrence_seq_ex(st_s, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                              dev(p["beta"]), y_s, scale)
    assert_close(host(y_s), y_ref, "sequential y, infinite decay")
    assert_close(host(st_s), st_ref, "sequential state, infinite decay")


def test_degenerate_inputs_both_scans():
    """Degenerate values the method admits, through the chunked and the
    sequential scan against the oracle: beta = 0 on a whole head (the state
    only decays), zero k at some positions (the L2 norm of a zero vector),
    zero q, g = 0 (no decay), and a head whose k is the same unit vector at
    every position (every off-diagonal entry of a chunk's A is nonzero)."""
    rng = np.random.default_rng(905)
    N, T, HK, H = 1, 150, 4, 4
    p = _case(rng, N, T, HK, H)
    p["beta"][:, :, 0] = 0.0
    for key in ("kh", "k"):
        p[key][:, 10:14, 1] = 0.0
        p[key][:, :, 3] = p[key][:, :1, 3]
    for key in ("qh", "q"):
        p[key][:, 70:90, 2] = 0.0
    p["g"][:, 30:100, 1] = 0.0
    scale = 1 / math.sqrt(128)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"],
                                          scale)
    y, st = _gpu_chunked(p, scale)
    assert_close(host(y), y_ref, "chunked y, degenerate inputs")
    assert_close(host(st), st_ref, "chunked state, degenerate inputs")
    st_s = dev(p["state"])
    y_s = torch.empty_like(y)
    gdn.gdn_recurrence_seq_ex(st_s, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                              dev(p["beta"]), y_s, scale)
    assert_close(host(y_s), y_ref, "sequential y, degenerate inputs")
    assert_close(host(st_s), st_ref, "sequential state, degenerate inputs")
