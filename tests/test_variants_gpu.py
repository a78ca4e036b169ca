"""Parity of the extended entry points (needs an MI355X): the "T4" read-out of
the decode, the grouped-query repeat done by index in decode and scan, and the
per-token snapshots of the scan and the conv for speculative decoding.

Each is checked against the oracle within the tolerance, and against the
plain entry points bit for bit where the arithmetic is the same.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, assert_close, dev, host, oracle_threads
from linear_attention_ssm_recurrence_amd import gdn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()
    oracle_threads()


def _inputs(rng, N, T, HK, H, S):
    """Recurrence inputs with K-head q/k (unit norm) and their tiled repeat."""
    qk = oracle.l2norm_gqa(rng.standard_normal((N, T, HK, S)), HK)
    kk = oracle.l2norm_gqa(rng.standard_normal((N, T, HK, S)), HK)
    rep = lambda x: np.ascontiguousarray(x[:, :, np.arange(H) % HK, :])
    v = rng.standard_normal((N, T, H, S)).astype(np.float32)
    g = oracle.decay_gate(rng.standard_normal((N, T, H)), np.zeros(H), rng.standard_normal(H))
    beta = oracle.sigmoid(rng.standard_normal((N, T, H)))
    st = (rng.standard_normal((N, H, S, S)) * 0.05).astype(np.float32)
    return dict(qh=qk, kh=kk, q=rep(qk), k=rep(kk), v=v, g=g, beta=beta, state=st)


@pytest.mark.parametrize("S", [32, 128, 256])
def test_decode_t4_and_gqa(S):
    rng = np.random.default_rng(500 + S)
    N, HK, H = 9, 4, 8
    p = _inputs(rng, N, 1, HK, H, S)
    scale = 1 / math.sqrt(S)
    sq = lambda x: np.ascontiguousarray(x[:, 0])
    y_ref, st_ref = oracle.recurrence(p["state"], sq(p["q"]), sq(p["k"]), sq(p["v"]), sq(p["g"]),
                                      sq(p["beta"]), scale)
    # exact read-out, repeat done by index == plain entry point on repeated q/k
    st_a, st_b, st_c = dev(p["state"]), dev(p["state"]), dev(p["state"])
    y_a = torch.empty((N, H, S), device=DEV)
    y_b = torch.empty_like(y_a)
    y_c = torch.empty_like(y_a)
    gdn.gdn_recurrence(st_a, dev(sq(p["q"])), dev(sq(p["k"])), dev(sq(p["v"])), dev(sq(p["g"])),
                       dev(sq(p["beta"])), y_a, scale)
    gdn.gdn_recurrence_ex(st_b, dev(sq(p["qh"])), dev(sq(p["kh"])), dev(sq(p["v"])),
                          dev(sq(p["g"])), dev(sq(p["beta"])), y_b, scale, gdn.GDN_RECUR_EXACT)
    gdn.gdn_recurrence_ex(st_c, dev(sq(p["qh"])), dev(sq(p["kh"])), dev(sq(p["v"])),
                          dev(sq(p["g"])), dev(sq(p["beta"])), y_c, scale, gdn.GDN_RECUR_T4)
    assert torch.equal(st_a, st_b) and torch.equal(y_a, y_b), "index GQA != repeated q/k"
    # T4: identical state trajectory, y within the tolerance of the oracle
    assert torch.equal(st_a, st_c), "T4 changed the state"
    assert_close(host(y_c), y_ref, f"T4 y S={S}")
    assert_close(host(st_c), st_ref, f"T4 state S={S}")


@pytest.mark.parametrize("S,T", [(128, 70), (64, 5), (32, 130)])
def test_scan_gqa_and_snapshots(S, T):
    rng = np.random.default_rng(600 + S + T)
    N, HK, H = 2, 2, 4
    p = _inputs(rng, N, T, HK, H, S)
    scale = 1 / math.sqrt(S)
    # plain scan on repeated q/k
    st_a = dev(p["state"])
    y_a = torch.empty((N, T, H, S), device=DEV)
    gdn.gdn_recurrence_seq(st_a, dev(p["q"]), dev(p["k"]), dev(p["v"]), dev(p["g"]), dev(p["beta"]),
                           y_a, scale)
    # extended scan: K-head q/k, snapshots
    st_b = dev(p["state"])
    y_b = torch.empty_like(y_a)
    snaps = torch.full((N, T, H, S, S), float("nan"), device=DEV)
    gdn.gdn_recurrence_seq_ex(st_b, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                              dev(p["beta"]), y_b, scale, snaps)
    assert torch.equal(y_a, y_b) and torch.equal(st_a, st_b), "index GQA != repeated q/k"
    assert torch.equal(snaps[:, T - 1], st_b), "last snapshot != final state"
    # every snapshot equals the state after that prefix (bits), for a sample of t
    for t in sorted({0, 1, T // 2, min(63, T - 1), min(64, T - 1), T - 1}):
        st_t = dev(p["state"])
        y_t = torch.empty((N, t + 1, H, S), device=DEV)
        gdn.gdn_recurrence_seq(st_t, dev(p["q"][:, :t + 1]), dev(p["k"][:, :t + 1]),
                               dev(p["v"][:, :t + 1]), dev(p["g"][:, :t + 1]),
                               dev(p["beta"][:, :t + 1]), y_t, scale)
        assert torch.equal(snaps[:, t], st_t), f"snapshot {t} != state after {t + 1} tokens"
    # and against the oracle, all tokens
    s = p["state"]
    sn = host(snaps)
    for t in range(T):
        _, s = oracle.recurrence(s, p["q"][:, t], p["k"][:, t], p["v"][:, t], p["g"][:, t],
                                 p["beta"][:, t], scale)
        if t % max(1, T // 8) == 0 or t == T - 1:
            assert_close(sn[:, t], s, f"snapshot {t} vs oracle")


@pytest.mark.parametrize("K,T", [(4, 37), (3, 2), (2, 17)])
def test_conv_snapshots(K, T):
    rng = np.random.default_rng(700 + K + T)
    N, C = 2, 300
    x = rng.standard_normal((N, T, C)).astype(np.float32)
    w = (rng.standard_normal((C, K)) * 0.5).astype(np.float32)
    cs0 = rng.standard_normal((N, C, K - 1)).astype(np.float32)
    out_ref, cs_ref = oracle.conv1d_silu_seq(x, w, cs0)
    cs = dev(cs0)
    out = torch.empty((N, T, C), device=DEV)
    snaps = torch.full((N, T, C, K - 1), float("nan"), device=DEV)
    gdn.gdn_conv1d_silu_seq_ex(dev(x), dev(w), cs, out, snaps)
    assert_close(host(out), out_ref, "conv out")
    assert np.array_equal(host(cs), cs_ref)
    sn = host(snaps)
    # history after position t = the last K-1 entries of (initial history ++ x[:t+1])
    full = np.concatenate([cs0, np.transpose(x, (0, 2, 1))], axis=2)   # [N][C][K-1+T]
    for t in range(T):
        assert np.array_equal(sn[:, t], full[:, :, t + 1:t + K]), f"conv snapshot {t}"


def test_t4_full_batch():
    """The bench's decode_t4 shape (256 x 32 x 128, q/k per K-head): the T4
    read-out leaves the state bit-identical to the exact read-out, and its y
    agrees with the exact y (which the full-batch parity test checks against
    the oracle) within the tolerance."""
    rng = np.random.default_rng(1700)
    N, HK, H, S = 256, 16, 32, 128
    qh = oracle.l2norm_gqa(rng.standard_normal((N, HK, S)), HK)
    kh = oracle.l2norm_gqa(rng.standard_normal((N, HK, S)), HK)
    v = rng.standard_normal((N, H, S)).astype(np.float32)
    g = oracle.decay_gate(rng.standard_normal((N, H)), np.zeros(H), rng.standard_normal(H))
    beta = oracle.sigmoid(rng.standard_normal((N, H)))
    st0 = (rng.standard_normal((N, H, S, S)) * 0.05).astype(np.float32)
    scale = 1 / math.sqrt(S)
    out = []
    for variant in (gdn.GDN_RECUR_EXACT, gdn.GDN_RECUR_T4):
        st = dev(st0)
        y = torch.empty((N, H, S), device=DEV)
        gdn.gdn_recurrence_ex(st, dev(qh), dev(kh), dev(v), dev(g), dev(beta), y, scale, variant)
        out.append((st, y))
    assert torch.equal(out[0][0], out[1][0]), "T4 changed the state"
    assert_close(host(out[1][1]), host(out[0][1]), "T4 y vs exact y, full batch")


def test_spec_verify_shape_snapshots():
    """The bench's speculative-verify shape (64 sequences x 4 tokens, 16 -> 32
    heads, S = 128): snapshot t equals the state after t + 1 decode launches,
    bit for bit, and the y of each token equals that launch's y."""
    rng = np.random.default_rng(1701)
    N, T, HK, H, S = 64, 4, 16, 32, 128
    p = _inputs(rng, N, T, HK, H, S)
    scale = 1 / math.sqrt(S)
    st = dev(p["state"])
    y = torch.empty((N, T, H, S), device=DEV)
    snaps = torch.full((N, T, H, S, S), float("nan"), device=DEV)
    gdn.gdn_recurrence_seq_ex(st, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                              dev(p["beta"]), y, scale, snaps)
    st_d = dev(p["state"])
    for t in range(T):
        y_d = torch.empty((N, H, S), device=DEV)
        sl = lambda x: dev(np.ascontiguousarray(x[:, t]))
        gdn.gdn_recurrence_ex(st_d, sl(p["qh"]), sl(p["kh"]), sl(p["v"]), sl(p["g"]),
                              sl(p["beta"]), y_d, scale, gdn.GDN_RECUR_EXACT)
        assert torch.equal(snaps[:, t], st_d), f"snapshot {t} != state after {t + 1} launches"
        assert torch.equal(y[:, t], y_d), f"y of token {t} != decode launch {t}"
    assert torch.equal(st, st_d)


def test_scan_many_blocks_short_chunks():
    """3 sequences x 70 tokens, 8 -> 32 heads, S = 128: 768 scan blocks, more
    than the CUs, which selects the 32-token chunk variant of the scan. It
    must match the oracle, and equal chained decode launches bit for bit."""
    rng = np.random.default_rng(1702)
    N, T, HK, H, S = 3, 70, 8, 32, 128
    p = _inputs(rng, N, T, HK, H, S)
    scale = 1 / math.sqrt(S)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"],
                                          scale)
    st = dev(p["state"])
    y = torch.empty((N, T, H, S), device=DEV)
    gdn.gdn_recurrence_seq_ex(st, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                              dev(p["beta"]), y, scale)
    assert_close(host(y), y_ref, "scan 768 blocks y")
    assert_close(host(st), st_ref, "scan 768 blocks state")
    st_d = dev(p["state"])
    for t in range(T):
        y_d = torch.empty((N, H, S), device=DEV)
        sl = lambda x: dev(np.ascontiguousarray(x[:, t]))
        gdn.gdn_recurrence_ex(st_d, sl(p["qh"]), sl(p["kh"]), sl(p["v"]), sl(p["g"]),
                              sl(p["beta"]), y_d, scale, gdn.GDN_RECUR_EXACT)
        assert torch.equal(y[:, t], y_d), f"token {t}: scan y != decode launch y"
    assert torch.equal(st, st_d), "scan state != chained decode launches"


def _scan_t4_case(seed, N, T, HK, H, S, with_snaps):
    """The scan with the "T4" read-out: y against the oracle within the
    tolerance and against gdn_recurrence_ex(GDN_RECUR_T4) applied token by
    token bit for bit; the state (and the snapshots) against the exact scan
    bit for bit, since only y is regrouped."""
    rng = np.random.default_rng(seed)
    p = _inputs(rng, N, T, HK, H, S)
    scale = 1 / math.sqrt(S)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"],
                                          scale)
    args = [dev(p[x]) for x in ("qh", "kh", "v", "g", "beta")]
    st_t4, st_ex = dev(p["state"]), dev(p["state"])
    y_t4 = torch.empty((N, T, H, S), device=DEV)
    y_ex = torch.empty_like(y_t4)
    sn_t4 = torch.empty((N, T, H, S, S), device=DEV) if with_snaps else None
    sn_ex = torch.empty_like(sn_t4) if with_snaps else None
    gdn.gdn_recurrence_seq_ex(st_t4, *args, y_t4, scale, sn_t4, variant=gdn.GDN_RECUR_T4)
    gdn.gdn_recurrence_seq_ex(st_ex, *args, y_ex, scale, sn_ex, variant=gdn.GDN_RECUR_EXACT)
    what = f"T4 scan N={N} T={T} HK={HK} H={H} S={S}"
    assert_close(host(y_t4), y_ref, what + " y")
    assert_close(host(st_t4), st_ref, what + " state")
    assert torch.equal(st_t4, st_ex), what + ": state differs from the exact scan"
    if with_snaps:
        assert torch.equal(sn_t4, sn_ex), what + ": snapshots differ from the exact scan"
    st_d = dev(p["state"])
    for t in range(T):
        y_d = torch.empty((N, H, S), device=DEV)
        sl = lambda x: dev(np.ascontiguousarray(p[x][:, t]))
        gdn.gdn_recurrence_ex(st_d, sl("qh"), sl("kh"), sl("v"), sl("g"), sl("beta"), y_d, scale,
                              gdn.GDN_RECUR_T4)
        assert torch.equal(y_t4[:, t], y_d), f"{what}: token {t} differs from the T4 decode"
    assert torch.equal(st_t4, st_d), what + ": state differs from chained T4 decodes"


@pytest.mark.parametrize("S", [32, 64, 128, 256])
@pytest.mark.parametrize("T", [5, 70])
def test_scan_t4(S, T):
    """T = 5 takes the short scan (decode layout, no LDS), T = 70 the chunked
    LDS scan with a ragged last chunk; k . q is formed in one shared order."""
    _scan_t4_case(600 + S + T, 2, T, 2, 4, S, with_snaps=(T == 5))


def test_scan_t4_many_blocks():
    """768 scan blocks: the 32-token chunk variant, GQA 8 -> 32."""
    _scan_t4_case(611, 3, 70, 8, 32, 128, with_snaps=False)
