"""Parity of the chained bf16 prefill (gdn_prefill_bf16, and gdn_prefill_bf16_ex
with either scan) with the oracle, and with the fused decode layer applied
position by position (needs an MI355X)."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, RTOL_LONG_SCAN, assert_close, dev_ssm_a, dev, dev_bits, host, oracle_threads
from linear_attention_ssm_recurrence_amd import gdn, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()
    oracle_threads()


SCANS = [None, gdn.GDN_SCAN_CHUNKED]


def _gpu_prefill(d, HK, scale, eps=1e-6, scan=None):
    N, T, H, S = d["z"].shape
    cs, st = dev(d["conv_state"]), dev(d["state"])
    out = torch.empty((N, T, H, S), device=DEV)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(N, T, HK, H, S), dtype=torch.uint8, device=DEV)
    gdn.gdn_prefill_bf16(dev_bits(d["qkv"]), dev_bits(d["z"]), dev(d["a"]), dev(d["b"]),
                         dev(d["conv_w"]), dev_ssm_a(d["A_log"]), dev(d["dt_bias"]), dev(d["norm_w"]),
                         cs, st, out, ws, HK, scale, eps, eps, scan=scan)
    return out, cs, st


def _oracle_prefill(d, HK, scale):
    return oracle.prefill_bf16(d["qkv"], d["z"], d["a"], d["b"], d["conv_w"], d["A_log"],
                               d["dt_bias"], d["norm_w"], d["conv_state"], d["state"], HK, scale)


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("N,T,HK,H,K", [(2, 37, 2, 4, 4), (1, 5, 1, 2, 2), (3, 16, 4, 4, 3),
                                         (2, 70, 2, 8, 4), (1, 130, 2, 4, 4)])
def test_prefill_small(N, T, HK, H, K, scan):
    d = inputs.draw_prefill(seed=100 + T, n_seqs=N, n_tokens=T, n_k_heads=HK, n_v_heads=H,
                            conv_kernel=K, state_sigma=0.05, conv_state_sigma=1.0)
    scale = 1 / math.sqrt(128)
    out, cs, st = _gpu_prefill(d, HK, scale, scan=scan)
    o_ref, cs_ref, st_ref = _oracle_prefill(d, HK, scale)
    assert_close(host(out), o_ref, f"prefill out N={N} T={T}")
    assert_close(host(st), st_ref, f"prefill state N={N} T={T}")
    assert np.array_equal(host(cs), cs_ref), "prefill conv history"


def test_prefill_equals_decode_layers():
    """T positions through gdn_prefill_bf16 == T calls of gdn_decode_block_bf16 (bits)."""
    N, T, HK, H, S = 3, 20, 2, 4, 128
    d = inputs.draw_prefill(seed=9, n_seqs=N, n_tokens=T, n_k_heads=HK, n_v_heads=H,
                            state_sigma=0.05, conv_state_sigma=1.0)
    scale = 1 / math.sqrt(S)
    out, cs, st = _gpu_prefill(d, HK, scale)
    cs2, st2 = dev(d["conv_state"]), dev(d["state"])
    for t in range(T):
        o = torch.empty((N, H, S), device=DEV)
        gdn.gdn_decode_block_bf16(dev_bits(np.ascontiguousarray(d["qkv"][:, t])),
                                  dev_bits(np.ascontiguousarray(d["z"][:, t])),
                                  dev(d["a"][:, t]), dev(d["b"][:, t]), dev(d["conv_w"]),
                                  dev_ssm_a(d["A_log"]), dev(d["dt_bias"]), dev(d["norm_w"]), cs2, st2,
                                  o, HK, scale, 1e-6, 1e-6)
        assert torch.equal(o, out[:, t]), f"position {t}: prefill != decode layer"
    assert torch.equal(st2, st) and torch.equal(cs2, cs)
    # the _ex entry point with the sequential scan is the same computation
    out3, cs3, st3 = _gpu_prefill(d, HK, scale, scan=gdn.GDN_SCAN_SEQUENTIAL)
    assert torch.equal(out3, out) and torch.equal(st3, st) and torch.equal(cs3, cs)


@pytest.mark.parametrize("scan", SCANS)
def test_prefill_4096_full(scan):
    """1 sequence x 4096 positions, 16 -> 32 heads, S = 128, C = 8192, K = 4."""
    d = inputs.draw_prefill()
    scale = 1 / math.sqrt(128)
    out, cs, st = _gpu_prefill(d, 16, scale, scan=scan)
    o_ref, cs_ref, st_ref = _oracle_prefill(d, 16, scale)
    assert_close(host(out), o_ref, "prefill 4096 out", rtol=RTOL_LONG_SCAN)
    assert_close(host(st), st_ref, "prefill 4096 state", rtol=RTOL_LONG_SCAN)
    assert np.array_equal(host(cs), cs_ref)
