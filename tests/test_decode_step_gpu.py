"""One decode step from raw inputs in one launch (gdn_decode_step) against the
oracle and, bit for bit, against the staged kernels it folds together
(gdn_l2norm_gqa for q and k, gdn_decay_gate, gdn_sigmoid, gdn_recurrence_ex),
through the C ABI (needs an MI355X): every state size, grouped-query ratios
1/2/4, chained steps on the same state, the full 256-sequence batch, and
zero q/k vectors (the eps floor of the norm)."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, assert_close, dev_ssm_a, dev, host, oracle_threads
from linear_attention_ssm_recurrence_amd import gdn, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()
    oracle_threads()


def _draw(rng, N, HK, H, S):
    return dict(q=rng.standard_normal((N, HK, S)).astype(np.float32),
                k=rng.standard_normal((N, HK, S)).astype(np.float32),
                v=rng.standard_normal((N, H, S)).astype(np.float32),
                a=rng.standard_normal((N, H)).astype(np.float32),
                b=rng.standard_normal((N, H)).astype(np.float32))


def _check_steps(N, HK, H, S, steps, seed, zero_qk=False, extreme_gate=False, l2_eps=1e-6):
    rng = np.random.default_rng(seed)
    A_log = rng.standard_normal(H).astype(np.float32)
    dt_bias = (0.5 * rng.standard_normal(H)).astype(np.float32)
    state0 = (0.05 * rng.standard_normal((N, H, S, S))).astype(np.float32)
    scale = 1 / math.sqrt(S)
    st_fused, st_staged = dev(state0), dev(state0)
    st_ref = state0
    for t in range(steps):
        x = _draw(rng, N, HK, H, S)
        if zero_qk:
            x["q"][:, 0] = 0.0
            x["k"][:, -1] = 0.0
        if extreme_gate:   # decay 0 and 1 in fp32, the softplus guard, saturated sigmoids
            x["a"][0, :6] = [1e30, -1e30, 20.0, np.nextafter(np.float32(20), np.float32(21)),
                             -80.0, 0.0]
            x["b"][0, :6] = [1e30, -1e30, 60.0, -60.0, 0.0, 1.0]
        d = {key: dev(val) for key, val in x.items()}
        Al, db = dev_ssm_a(A_log), dev(dt_bias)
        y = torch.empty((N, H, S), device=DEV)
        gdn.gdn_decode_step(st_fused, d["q"], d["k"], d["v"], d["a"], d["b"], Al, db, y, scale,
                            l2_eps)
        qs = torch.empty((N, H, S), device=DEV)
        ks = torch.empty((N, H, S), device=DEV)
        g = torch.empty((N, H), device=DEV)
        beta = torch.empty((N, H), device=DEV)
        gdn.gdn_l2norm_gqa(d["q"], qs, l2_eps)
        gdn.gdn_l2norm_gqa(d["k"], ks, l2_eps)
        gdn.gdn_decay_gate(d["a"], db, Al, g)
        gdn.gdn_sigmoid(d["b"], beta)
        y2 = torch.empty((N, H, S), device=DEV)
        gdn.gdn_recurrence(st_staged, qs, ks, d["v"], g, beta, y2, scale)
        what = f"N={N} HK={HK} H={H} S={S} step {t}"
        torch.cuda.synchronize()
        assert torch.equal(y, y2), f"{what}: fused y != staged y (bits)"
        assert torch.equal(st_fused, st_staged), f"{what}: fused state != staged state (bits)"
        qr = oracle.l2norm_gqa(x["q"], H, l2_eps)
        kr = oracle.l2norm_gqa(x["k"], H, l2_eps)
        gr = oracle.decay_gate(x["a"], dt_bias, A_log)
        br = oracle.sigmoid(x["b"])
        y_ref, st_ref = oracle.recurrence(st_ref, qr, kr, x["v"], gr, br, scale)
        assert_close(host(y), y_ref, f"{what} y")
        assert_close(host(st_fused), st_ref, f"{what} state")


@pytest.mark.parametrize("S", [32, 64, 128, 256])
@pytest.mark.parametrize("GQ", [1, 2, 4])
def test_decode_step_shapes(S, GQ):
    _check_steps(N=3, HK=2, H=2 * GQ, S=S, steps=3, seed=S * 10 + GQ)


def test_decode_step_zero_qk():
    """q or k of a K-head all zero: the norm's eps floor gives a zero vector."""
    _check_steps(N=2, HK=4, H=8, S=128, steps=2, seed=7, zero_qk=True)


def test_decode_step_extreme_gate_inputs():
    _check_steps(N=2, HK=4, H=8, S=128, steps=2, seed=8, extreme_gate=True)


def test_decode_step_256_sequences():
    """The batched decode workload: 256 sequences, 16 -> 32 heads, S = 128."""
    w = inputs.WORKLOADS[2]
    _check_steps(N=w.n_seqs, HK=w.n_k_heads, H=w.n_v_heads, S=w.state_size, steps=1, seed=11)


def test_decode_step_empty_is_noop():
    assert gdn.load_library().gdn_decode_step(
        None, None, None, None, None, None, None, None, None, 0, 16, 32, 128, 0.1, 1e-6,
        None) == gdn.GDN_OK
