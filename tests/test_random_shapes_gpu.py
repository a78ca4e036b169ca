"""Seeded random shapes for every entry point family, each against the oracle
within the tolerance (needs an MI355X).

The fixed-shape parity files cover the workloads at their real sizes; this
sweep draws many small, odd shapes (sequence, token and head counts, state
sizes, conv widths, grouped-query ratios, head dims) from fixed seeds, so that
ragged tails and unusual combinations are exercised too. The fused decode
layer's family runs both of its kernels (one workgroup per K-head, and 64-row
workgroups) on each case.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, assert_close, dev_ssm_a, dev, dev_bits, host, oracle_threads
from linear_attention_ssm_recurrence_amd import gdn, inputs

pytestmark = pytest.mark.gpu
CASES = range(64)


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()
    oracle_threads()


def _recurrence_inputs(rng, N, T, HK, H, S):
    qh = oracle.l2norm_gqa(rng.standard_normal((N, T, HK, S)), HK)
    kh = oracle.l2norm_gqa(rng.standard_normal((N, T, HK, S)), HK)
    rep = lambda x: np.ascontiguousarray(x[:, :, np.arange(H) % HK, :])
    return dict(
        qh=qh, kh=kh, q=rep(qh), k=rep(kh),
        v=rng.standard_normal((N, T, H, S)).astype(np.float32),
        g=oracle.decay_gate(rng.standard_normal((N, T, H)), rng.standard_normal(H) * 0.5,
                            rng.standard_normal(H)),
        beta=oracle.sigmoid(rng.standard_normal((N, T, H))),
        state=(rng.standard_normal((N, H, S, S)) * 0.05).astype(np.float32))


@pytest.mark.parametrize("case", CASES)
def test_random_decode(case):
    rng = np.random.default_rng(10_000 + case)
    S = int(rng.choice([32, 64, 128, 256]))
    HK = int(rng.choice([1, 2, 4]))
    H = HK * int(rng.choice([1, 2, 4]))
    N = int(rng.integers(1, 40))
    variant = int(rng.integers(0, 2))
    p = _recurrence_inputs(rng, N, 1, HK, H, S)
    scale = 1 / math.sqrt(S)
    sq = lambda x: np.ascontiguousarray(x[:, 0])
    y_ref, st_ref = oracle.recurrence(p["state"], sq(p["q"]), sq(p["k"]), sq(p["v"]), sq(p["g"]),
                                      sq(p["beta"]), scale)
    st = dev(p["state"])
    y = torch.empty((N, H, S), device=DEV)
    gdn.gdn_recurrence_ex(st, dev(sq(p["qh"])), dev(sq(p["kh"])), dev(sq(p["v"])), dev(sq(p["g"])),
                          dev(sq(p["beta"])), y, scale, variant)
    what = f"decode N={N} HK={HK} H={H} S={S} variant={variant}"
    assert_close(host(y), y_ref, what + " y")
    assert_close(host(st), st_ref, what + " state")


@pytest.mark.parametrize("case", CASES)
def test_random_scan(case):
    rng = np.random.default_rng(11_000 + case)
    S = int(rng.choice([32, 64, 128, 256]))
    HK = int(rng.choice([1, 2]))
    H = HK * int(rng.choice([1, 2]))
    N = int(rng.integers(1, 3))
    T = int(rng.integers(1, 150 if S <= 128 else 40))
    snap = bool(rng.integers(0, 2)) and N * T * H * S * S <= (1 << 22)
    variant = int(rng.integers(0, 2))       # exact or "T4" read-out
    p = _recurrence_inputs(rng, N, T, HK, H, S)
    scale = 1 / math.sqrt(S)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"],
                                          scale)
    st = dev(p["state"])
    y = torch.empty((N, T, H, S), device=DEV)
    snaps = torch.empty((N, T, H, S, S), device=DEV) if snap else None
    gdn.gdn_recurrence_seq_ex(st, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                              dev(p["beta"]), y, scale, snaps, variant=variant)
    what = f"scan N={N} T={T} HK={HK} H={H} S={S} snaps={snap} variant={variant}"
    assert_close(host(y), y_ref, what + " y")
    assert_close(host(st), st_ref, what + " state")
    if snap:
        assert torch.equal(snaps[:, T - 1], st), what + " last snapshot"


@pytest.mark.parametrize("case", CASES)
def test_random_chunked(case):
    rng = np.random.default_rng(12_000 + case)
    HK = int(rng.choice([1, 2, 4]))
    H = HK * int(rng.choice([1, 2, 3, 4, 8]))   # group sizes that split over blocks, or not
    N = int(rng.integers(1, 3))
    T = int(rng.integers(1, 300))
    S = 128
    p = _recurrence_inputs(rng, N, T, HK, H, S)
    scale = 1 / math.sqrt(S)
    y_ref, st_ref = oracle.recurrence_seq(p["state"], p["q"], p["k"], p["v"], p["g"], p["beta"],
                                          scale)
    st = dev(p["state"])
    y = torch.empty((N, T, H, S), device=DEV)
    ws = torch.empty(gdn.gdn_chunked_workspace_bytes(N, T, H, S), dtype=torch.uint8, device=DEV)
    gdn.gdn_recurrence_seq_chunked(st, dev(p["qh"]), dev(p["kh"]), dev(p["v"]), dev(p["g"]),
                                   dev(p["beta"]), y, scale, ws)
    what = f"chunked N={N} T={T} HK={HK} H={H}"
    assert_close(host(y), y_ref, what + " y")
    assert_close(host(st), st_ref, what + " state")


@pytest.mark.parametrize("case", CASES)
def test_random_conv(case):
    rng = np.random.default_rng(13_000 + case)
    K = int(rng.choice([2, 3, 4]))
    N = int(rng.integers(1, 4))
    T = int(rng.integers(1, 100))
    C = int(rng.integers(1, 700))
    x = rng.standard_normal((N, T, C)).astype(np.float32)
    w = (rng.standard_normal((C, K)) * 0.5).astype(np.float32)
    cs0 = rng.standard_normal((N, C, K - 1)).astype(np.float32)
    out_ref, cs_ref = oracle.conv1d_silu_seq(x, w, cs0)
    cs = dev(cs0)
    out = torch.empty((N, T, C), device=DEV)
    gdn.gdn_conv1d_silu_seq(dev(x), dev(w), cs, out)
    what = f"conv N={N} T={T} C={C} K={K}"
    assert_close(host(out), out_ref, what + " out")
    assert np.array_equal(host(cs), cs_ref), what + " history"


@pytest.mark.parametrize("case", CASES)
def test_random_prefill(case):
    rng = np.random.default_rng(14_000 + case)
    HK = int(rng.choice([1, 2, 4]))
    H = HK * int(rng.choice([1, 2]))
    N = int(rng.integers(1, 3))
    T = int(rng.integers(1, 100))
    K = int(rng.choice([2, 3, 4]))
    scan = [None, gdn.GDN_SCAN_CHUNKED][case % 2]
    d = inputs.draw_prefill(seed=15_000 + case, n_seqs=N, n_tokens=T, n_k_heads=HK, n_v_heads=H,
                            conv_kernel=K, state_sigma=0.05, conv_state_sigma=1.0)
    scale = 1 / math.sqrt(128)
    o_ref, cs_ref, st_ref = oracle.prefill_bf16(d["qkv"], d["z"], d["a"], d["b"], d["conv_w"],
                                                d["A_log"], d["dt_bias"], d["norm_w"],
                                                d["conv_state"], d["state"], HK, scale)
    cs, st = dev(d["conv_state"]), dev(d["state"])
    out = torch.empty((N, T, H, 128), device=DEV)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(N, T, HK, H, 128), dtype=torch.uint8,
                     device=DEV)
    gdn.gdn_prefill_bf16(dev_bits(d["qkv"]), dev_bits(d["z"]), dev(d["a"]), dev(d["b"]),
                         dev(d["conv_w"]), dev_ssm_a(d["A_log"]), dev(d["dt_bias"]), dev(d["norm_w"]),
                         cs, st, out, ws, HK, scale, scan=scan)
    what = f"prefill N={N} T={T} HK={HK} H={H} K={K} scan={scan}"
    assert_close(host(out), o_ref, what + " out")
    assert_close(host(st), st_ref, what + " state")
    assert np.array_equal(host(cs), cs_ref), what + " history"


@pytest.mark.parametrize("case", CASES)
def test_random_norms(case):
    rng = np.random.default_rng(16_000 + case)
    D = int(rng.choice([32, 64, 96, 128, 256, 1024]))
    rows = int(rng.integers(1, 500))
    y = rng.standard_normal((rows, D)).astype(np.float32)
    z = rng.standard_normal((rows, D)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    out = torch.empty((rows, D), device=DEV)
    gdn.gdn_gated_rmsnorm(dev(y), dev(w), dev(z), out, 1e-6)
    assert_close(host(out), oracle.gated_rmsnorm(y, w, z), f"gated norm rows={rows} D={D}")
    HK = int(rng.choice([1, 2, 4]))
    H = HK * int(rng.choice([1, 2, 4]))
    n = int(rng.integers(1, 60))
    x = rng.standard_normal((n, HK, D)).astype(np.float32)
    if case % 3 == 0:
        x[0] *= 1e-9                          # below the eps floor
    got = torch.empty((n, H, D), device=DEV)
    gdn.gdn_l2norm_gqa(dev(x), got, 1e-6)
    assert_close(host(got), oracle.l2norm_gqa(x, H, 1e-6), f"l2norm n={n} HK={HK} H={H} D={D}")


@pytest.mark.parametrize("case", CASES)
def test_random_decode_layer(case):
    """Both fused decode layers on a random batch: the one-workgroup layer and
    the layer split over 64-row workgroups, each against the oracle, and the
    two bit for bit; the split layer's workspace is zero again afterwards."""
    rng = np.random.default_rng(70_000 + case)
    S = 128
    HK = int(rng.integers(1, 7))
    GQ = int(rng.choice([1, 2, 4]))
    H = HK * GQ
    K = int(rng.integers(2, 5))
    N = int(rng.integers(1, 24))
    C = 2 * HK * S + H * S
    bits = lambda x: inputs.to_bf16_bits(x.astype(np.float32))
    d = dict(qkv=bits(rng.standard_normal((N, C))), z=bits(rng.standard_normal((N, H, S))),
             a=rng.standard_normal((N, H)).astype(np.float32),
             b=rng.standard_normal((N, H)).astype(np.float32),
             conv_w=(rng.standard_normal((C, K)) * 0.5).astype(np.float32),
             A_log=rng.standard_normal(H).astype(np.float32),
             dt_bias=(0.5 * rng.standard_normal(H)).astype(np.float32),
             norm_w=(1 + 0.1 * rng.standard_normal(S)).astype(np.float32),
             conv_state=rng.standard_normal((N, C, K - 1)).astype(np.float32),
             state=(0.05 * rng.standard_normal((N, H, S, S))).astype(np.float32))
    scale = 1 / math.sqrt(S)
    o_ref, cs_ref, st_ref = oracle.decode_block_bf16(
        d["qkv"], d["z"], d["a"], d["b"], d["conv_w"], d["A_log"], d["dt_bias"], d["norm_w"],
        d["conv_state"], d["state"], HK, scale)
    fixed = [dev(d["conv_w"]), dev_ssm_a(d["A_log"]), dev(d["dt_bias"]), dev(d["norm_w"])]
    step = [dev_bits(d["qkv"]), dev_bits(d["z"]), dev(d["a"]), dev(d["b"])]
    ws = torch.zeros(gdn.gdn_decode_block_workspace_bytes(N, HK, H), dtype=torch.uint8, device=DEV)
    results = []
    for split in (False, True):
        cs, st = dev(d["conv_state"]), dev(d["state"])
        out = torch.empty((N, H, S), device=DEV)
        if split:
            gdn.gdn_decode_block_bf16_ex(*step, *fixed, cs, st, out, ws, HK, scale)
        else:
            gdn.gdn_decode_block_bf16(*step, *fixed, cs, st, out, HK, scale)
        what = f"case {case} (N={N}, HK={HK}, GQ={GQ}, K={K}, split={split})"
        assert_close(host(out), o_ref, f"{what} out")
        assert_close(host(st), st_ref, f"{what} state")
        assert np.array_equal(host(cs), cs_ref), f"{what} conv history"
        results.append((out, st, cs))
    for a, b, name in zip(results[0], results[1], ("out", "state", "conv history")):
        assert torch.equal(a, b), f"case {case}: split layer != one-workgroup layer ({name} bits)"
    assert int(ws.count_nonzero()) == 0, f"case {case}: workspace not zero after the call"
