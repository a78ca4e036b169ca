"""The fused decode layer split over 64-row workgroups (gdn_decode_block_bf16_ex)
against the oracle and, bit for bit, against the one-workgroup-per-K-head layer
(gdn_decode_block_bf16), through the C ABI (needs an MI355X).

The split layer finds the last workgroup of each (sequence, K-head) and of
each (sequence, V-head) through counters in a caller-owned workspace, and
leaves that workspace zero. Each test checks the results after every call and
that the workspace is zero again, over chained calls on the same buffers, with
group counts that do and do not fill the launch grid's last row of eight
workgroup groups, every supported group size and conv width, and a workspace
reused at a smaller batch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, assert_close, dev_ssm_a, dev, dev_bits, host, oracle_threads
from linear_attention_ssm_recurrence_amd import gdn, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()
    oracle_threads()


def _workspace(N, HK, H):
    return torch.zeros(gdn.gdn_decode_block_workspace_bytes(N, HK, H), dtype=torch.uint8,
                       device=DEV)


def _rand_layer(rng, N, HK, GQ, K, S=128):
    H = GQ * HK
    C = 2 * HK * S + H * S
    bits = lambda x: inputs.to_bf16_bits(x.astype(np.float32))
    return dict(qkv=bits(rng.standard_normal((N, C))), z=bits(rng.standard_normal((N, H, S))),
                a=rng.standard_normal((N, H)).astype(np.float32),
                b=rng.standard_normal((N, H)).astype(np.float32),
                conv_w=(rng.standard_normal((C, K)) * 0.5).astype(np.float32),
                A_log=rng.standard_normal(H).astype(np.float32),
                dt_bias=(0.1 * rng.standard_normal(H)).astype(np.float32),
                norm_w=(1 + 0.1 * rng.standard_normal(S)).astype(np.float32),
                conv_state=rng.standard_normal((N, C, K - 1)).astype(np.float32),
                state=(0.05 * rng.standard_normal((N, H, S, S))).astype(np.float32))


def _rand_step(rng, N, H, S, C):
    """Per-call activations of one decode step: qkv, z (bf16 patterns), a, b."""
    bits = lambda x: inputs.to_bf16_bits(x.astype(np.float32))
    return dict(qkv=bits(rng.standard_normal((N, C))), z=bits(rng.standard_normal((N, H, S))),
                a=rng.standard_normal((N, H)).astype(np.float32),
                b=rng.standard_normal((N, H)).astype(np.float32))


class _Pair:
    """The same layer's buffers twice on the device: one set for each entry point."""

    def __init__(self, d):
        self.fixed = {k: dev(d[k]) for k in ("conv_w", "dt_bias", "norm_w")}
        self.fixed["ssm_a"] = dev_ssm_a(d["A_log"])
        N, H, S = d["z"].shape
        self.one = {"conv_state": dev(d["conv_state"]), "state": dev(d["state"]),
                    "out": torch.empty((N, H, S), dtype=torch.float32, device=DEV)}
        self.split = {k: v.clone() for k, v in self.one.items()}

    def step(self, x, HK, scale, ws):
        """One call of each entry point on step inputs x (qkv, z, a, b)."""
        qkv, z, a, b = dev_bits(x["qkv"]), dev_bits(x["z"]), dev(x["a"]), dev(x["b"])
        f = self.fixed
        for bufs, fn, extra in ((self.one, gdn.gdn_decode_block_bf16, ()),
                                (self.split, gdn.gdn_decode_block_bf16_ex, (ws,))):
            fn(qkv, z, a, b, f["conv_w"], f["ssm_a"], f["dt_bias"], f["norm_w"],
               bufs["conv_state"], bufs["state"], bufs["out"], *extra, HK, scale, 1e-6, 1e-6)

    def assert_equal(self, what):
        torch.cuda.synchronize()
        for k in ("out", "state", "conv_state"):
            assert torch.equal(self.split[k], self.one[k]), \
                f"{what}: split layer != one-workgroup layer ({k} bits)"


def _oracle_step(d, x, HK, scale):
    return oracle.decode_block_bf16(x["qkv"], x["z"], x["a"], x["b"], d["conv_w"], d["A_log"],
                                    d["dt_bias"], d["norm_w"], d["conv_state"], d["state"], HK,
                                    scale, 1e-6, 1e-6)


def _run_chain(d, HK, steps, rng, what, ws=None):
    """steps chained calls on the same buffers; fresh qkv, z, a, b per step."""
    N, H, S = d["z"].shape
    scale = 1 / math.sqrt(S)
    ws = _workspace(N, HK, H) if ws is None else ws
    pair = _Pair(d)
    ref = {"conv_state": d["conv_state"], "state": d["state"]}
    for t in range(steps):
        x = ({k: d[k] for k in ("qkv", "z", "a", "b")} if t == 0
             else _rand_step(rng, N, H, S, d["conv_w"].shape[0]))
        pair.step(x, HK, scale, ws)
        o_ref, cs_ref, st_ref = _oracle_step({**d, **ref}, x, HK, scale)
        ref = {"conv_state": cs_ref, "state": st_ref}
        pair.assert_equal(f"{what} step {t}")
        assert int(ws.count_nonzero()) == 0, f"{what} step {t}: workspace not zero after the call"
        assert_close(host(pair.split["out"]), o_ref, f"{what} step {t} out")
        assert_close(host(pair.split["state"]), st_ref, f"{what} step {t} state")
        assert np.array_equal(host(pair.split["conv_state"]), cs_ref), f"{what} step {t} history"
    return ws


@pytest.mark.parametrize("layer", [0, 47])
def test_split_block_64_sequences(layer):
    """Layers of the 48-layer block workload: 64 sequences, 16 K-heads -> 32
    V-heads, S = 128, C = 8192, K = 4, as the benchmark launches it; two
    chained calls."""
    w = inputs.WORKLOADS[4]
    d = inputs.draw_block_layer(layer)
    _run_chain(d, w.n_k_heads, 2, np.random.default_rng(100 + layer), f"64 seqs layer {layer}")


@pytest.mark.parametrize("GQ", [1, 2, 4])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_split_block_shapes(GQ, K):
    """3 sequences x 3 K-heads: 9 groups, so the last row of eight groups is
    partly empty; three chained calls."""
    rng = np.random.default_rng(200 + GQ * 10 + K)
    d = _rand_layer(rng, 3, 3, GQ, K)
    _run_chain(d, 3, 3, rng, f"split GQ={GQ} K={K}")


def test_split_block_workspace_reused_smaller():
    """A workspace sized for 12 sequences, used for 12 and then for 5."""
    rng = np.random.default_rng(300)
    ws = _workspace(12, 16, 32)
    _run_chain(_rand_layer(rng, 12, 16, 2, 4), 16, 2, rng, "12 sequences", ws=ws)
    _run_chain(_rand_layer(rng, 5, 16, 2, 4), 16, 2, rng, "5 sequences", ws=ws)


def test_split_block_one_sequence():
    """One sequence, 16 -> 32 heads: 16 groups x 4 workgroups."""
    rng = np.random.default_rng(400)
    _run_chain(_rand_layer(rng, 1, 16, 2, 4), 16, 3, rng, "one sequence")


def test_split_block_empty_is_noop():
    assert gdn.load_library().gdn_decode_block_bf16_ex(
        None, None, None, None, None, None, None, None, None, None, None, None, 0,
        0, 16, 32, 128, 4, 0.1, 1e-6, 1e-6, None) == gdn.GDN_OK


def test_split_block_degenerate_inputs():
    """Zero activations and histories for some sequences (q and k fall to the
    eps floor of the L2 norm, the read-out and the norm's sum to zero), gate
    inputs at +-1e30 and on both sides of the softplus guard at 20 (decay 0 and
    1 to fp32), and beta inputs that saturate the sigmoid: bit for bit against
    the one-workgroup layer and within the tolerance of the oracle."""
    rng = np.random.default_rng(500)
    N, HK, GQ, K = 5, 3, 2, 4
    d = _rand_layer(rng, N, HK, GQ, K)
    H, S = HK * GQ, 128
    zero16 = inputs.to_bf16_bits(np.zeros(1, dtype=np.float32))[0]
    d["qkv"][1] = zero16                      # sequence 1: all conv inputs zero ...
    d["conv_state"][1] = 0.0                  # ... and no history: q = k = v = 0
    d["z"][2] = zero16                        # sequence 2: silu(z) = 0, out = 0
    d["a"][3] = np.array([1e30, -1e30, 20.0, np.nextafter(np.float32(20), np.float32(21)),
                          -80.0, 0.0], dtype=np.float32)[:H]
    d["b"][3] = np.array([1e30, -1e30, 60.0, -60.0, 0.0, 1.0], dtype=np.float32)[:H]
    d["state"][4] = 0.0                       # sequence 4: empty state
    _run_chain(d, HK, 1, rng, "degenerate inputs")
