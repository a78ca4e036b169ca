"""Out-of-range writes: every entry point, through the C ABI, writes into
output and in-place buffers that sit between guard regions of a known byte
pattern; after the call the guards (16 KiB before, and at least 16 KiB after
each buffer, including the slack that rounds a buffer up to 256 bytes) must
be unchanged. Sizes are ragged on purpose: token counts 5, 65, 70 and 130
against 16-, 32- and 64-position tiles; conv widths 2 to 4 over 1000
channels (not a multiple of a 256-thread block); head and sequence counts
that leave the split layer's last row of eight workgroup groups part-empty;
every state size; workspaces of exactly the size the library asks for
(needs an MI355X).
"""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, dev_ssm_a
from linear_attention_ssm_recurrence_amd import gdn

pytestmark = pytest.mark.gpu

GUARD = 16384
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


class Guarded:
    """A device buffer of `shape` and `dtype` inside guard bytes."""

    def __init__(self, shape, dtype=torch.float32, init=None):
        n = math.prod(shape) * torch.tensor([], dtype=dtype).element_size()
        self.nbytes = n
        padded = (n + 255) // 256 * 256
        self.raw = torch.full((GUARD + padded + GUARD,), PATTERN, dtype=torch.uint8, device=DEV)
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(shape)
        if init is not None:
            self.t.copy_(init)

    def check(self, what):
        torch.cuda.synchronize()
        lo = self.raw[:GUARD]
        hi = self.raw[GUARD + self.nbytes:]
        bad_lo = int((lo != PATTERN).sum())
        bad_hi = int((hi != PATTERN).sum())
        assert bad_lo == 0 and bad_hi == 0, \
            f"{what}: {bad_lo} guard bytes changed before the buffer, {bad_hi} after it"


def rnd(gen, *shape, sd=1.0):
    return torch.randn(shape, generator=gen, device=DEV) * sd


def bf16(x):
    return (x.view(torch.int32) >> 16).to(torch.int16)


@pytest.fixture
def gen():
    return torch.Generator(device=DEV).manual_seed(2024)


def test_pointwise(gen):
    al = rnd(gen, 37)
    s = Guarded((37,))
    gdn.gdn_ssm_a(al, s.t)
    s.check("gdn_ssm_a")
    ssm = dev_ssm_a(rnd(gen, 7))
    g = Guarded((33, 7))
    gdn.gdn_decay_gate(rnd(gen, 33, 7), rnd(gen, 7), ssm, g.t)
    g.check("gdn_decay_gate")
    y = Guarded((1001,))
    gdn.gdn_sigmoid(rnd(gen, 1001), y.t)
    y.check("gdn_sigmoid")
    o = Guarded((13, 6, 36))
    gdn.gdn_l2norm_gqa(rnd(gen, 13, 3, 36), o.t, 1e-6)
    o.check("gdn_l2norm_gqa")
    for D in (128, 96):
        out = Guarded((37, D))
        gdn.gdn_gated_rmsnorm(rnd(gen, 37, D), 1 + rnd(gen, D, sd=0.1), rnd(gen, 37, D), out.t,
                              1e-6)
        out.check(f"gdn_gated_rmsnorm D={D}")


@pytest.mark.parametrize("K", [2, 3, 4])
def test_conv(gen, K):
    N, C = 3, 1000
    cs = Guarded((N, C, K - 1), init=rnd(gen, N, C, K - 1))
    out = Guarded((N, C))
    gdn.gdn_conv1d_silu(rnd(gen, N, C), rnd(gen, C, K, sd=0.5), cs.t, out.t)
    cs.check(f"gdn_conv1d_silu K={K} conv_state")
    out.check(f"gdn_conv1d_silu K={K} out")
    for T in (5, 65, 70, 130):
        cs = Guarded((2, C, K - 1), init=rnd(gen, 2, C, K - 1))
        out = Guarded((2, T, C))
        snaps = Guarded((2, T, C, K - 1))
        gdn.gdn_conv1d_silu_seq_ex(rnd(gen, 2, T, C), rnd(gen, C, K, sd=0.5), cs.t, out.t,
                                   snaps.t)
        for b, name in ((cs, "conv_state"), (out, "out"), (snaps, "snaps")):
            b.check(f"gdn_conv1d_silu_seq_ex K={K} T={T} {name}")


def _rec_inputs(gen, N, T, HK, H, S):
    q = torch.nn.functional.normalize(rnd(gen, N, T, HK, S), dim=-1)
    k = torch.nn.functional.normalize(rnd(gen, N, T, HK, S), dim=-1)
    g = -torch.rand((N, T, H), generator=gen, device=DEV)
    b = torch.rand((N, T, H), generator=gen, device=DEV)
    return q, k, rnd(gen, N, T, H, S), g, b


@pytest.mark.parametrize("S", [32, 64, 128, 256])
def test_decode(gen, S):
    N, HK, H = 3, 2, 4
    q, k, v, g, b = (t[:, 0] for t in _rec_inputs(gen, N, 1, HK, H, S))
    for variant in (gdn.GDN_RECUR_EXACT, gdn.GDN_RECUR_T4):
        st = Guarded((N, H, S, S), init=rnd(gen, N, H, S, S, sd=0.05))
        y = Guarded((N, H, S))
        gdn.gdn_recurrence_ex(st.t, q, k, v, g, b, y.t, S ** -0.5, variant)
        st.check(f"gdn_recurrence_ex S={S} variant {variant} state")
        y.check(f"gdn_recurrence_ex S={S} variant {variant} y")
    st = Guarded((N, H, S, S), init=rnd(gen, N, H, S, S, sd=0.05))
    y = Guarded((N, H, S))
    gdn.gdn_decode_step(st.t, rnd(gen, N, HK, S), rnd(gen, N, HK, S), v, rnd(gen, N, H),
                        rnd(gen, N, H), dev_ssm_a(rnd(gen, H)), rnd(gen, H), y.t, S ** -0.5)
    st.check(f"gdn_decode_step S={S} state")
    y.check(f"gdn_decode_step S={S} y")


@pytest.mark.parametrize("T", [5, 65, 70, 130])
@pytest.mark.parametrize("S", [64, 128])
def test_scan(gen, T, S):
    N, HK, H = 2, 2, 4
    q, k, v, g, b = _rec_inputs(gen, N, T, HK, H, S)
    for variant in (gdn.GDN_RECUR_EXACT, gdn.GDN_RECUR_T4):
        st = Guarded((N, H, S, S), init=rnd(gen, N, H, S, S, sd=0.05))
        y = Guarded((N, T, H, S))
        snaps = Guarded((N, T, H, S, S))
        gdn.gdn_recurrence_seq_ex(st.t, q, k, v, g, b, y.t, S ** -0.5, snaps.t, variant=variant)
        for buf, name in ((st, "state"), (y, "y"), (snaps, "snaps")):
            buf.check(f"gdn_recurrence_seq_ex T={T} S={S} variant {variant} {name}")
    if S == 128:
        st = Guarded((N, H, S, S), init=rnd(gen, N, H, S, S, sd=0.05))
        y = Guarded((N, T, H, S))
        ws = Guarded((gdn.gdn_chunked_workspace_bytes(N, T, H, S),), dtype=torch.uint8)
        gdn.gdn_recurrence_seq_chunked(st.t, q, k, v, g, b, y.t, S ** -0.5, ws.t)
        for buf, name in ((st, "state"), (y, "y"), (ws, "workspace")):
            buf.check(f"gdn_recurrence_seq_chunked T={T} {name}")


def _layer(gen, N, HK, H, K, T=None, S=128):
    C = 2 * HK * S + H * S
    lead = (N,) if T is None else (N, T)
    return dict(qkv=bf16(rnd(gen, *lead, C)), z=bf16(rnd(gen, *lead, H, S)),
                a=rnd(gen, *lead, H), b=rnd(gen, *lead, H), conv_w=rnd(gen, C, K, sd=0.5),
                ssm_a=dev_ssm_a(rnd(gen, H)), dt_bias=rnd(gen, H, sd=0.1),
                norm_w=1 + rnd(gen, S, sd=0.1), conv_state=rnd(gen, N, C, K - 1),
                state=rnd(gen, N, H, S, S, sd=0.05))


@pytest.mark.parametrize("N,HK,GQ,K", [(3, 3, 2, 3), (1, 5, 1, 2), (2, 3, 4, 4)])
def test_decode_layers(gen, N, HK, GQ, K):
    H, S = HK * GQ, 128
    d = _layer(gen, N, HK, H, K)
    C = d["qkv"].shape[1]
    for form in ("one", "ex", "noalloc"):
        cs = Guarded((N, C, K - 1), init=d["conv_state"])
        st = Guarded((N, H, S, S), init=d["state"])
        out = Guarded((N, H, S))
        args = (d["qkv"], d["z"], d["a"], d["b"], d["conv_w"], d["ssm_a"], d["dt_bias"],
                d["norm_w"], cs.t, st.t, out.t)
        bufs = [(cs, "conv_state"), (st, "state"), (out, "out")]
        if form == "one":
            gdn.gdn_decode_block_bf16(*args, HK, S ** -0.5)
        elif form == "ex":
            ws = Guarded((gdn.gdn_decode_block_workspace_bytes(N, HK, H),), dtype=torch.uint8,
                         init=torch.zeros(gdn.gdn_decode_block_workspace_bytes(N, HK, H),
                                          dtype=torch.uint8, device=DEV))
            gdn.gdn_decode_block_bf16_ex(*args[:11], ws.t, HK, S ** -0.5)
            bufs.append((ws, "workspace"))
        else:
            gdn.gdn_decode_block_bf16_noalloc(*args, HK, S ** -0.5)
        for buf, name in bufs:
            buf.check(f"decode layer ({form}) N={N} HK={HK} GQ={GQ} K={K} {name}")


@pytest.mark.parametrize("T", [5, 70, 130])
def test_prefill(gen, T):
    N, HK, H, K, S = 2, 2, 4, 4, 128
    d = _layer(gen, N, HK, H, K, T=T)
    C = d["qkv"].shape[-1]
    for scan in (gdn.GDN_SCAN_SEQUENTIAL, gdn.GDN_SCAN_CHUNKED):
        cs = Guarded((N, C, K - 1), init=d["conv_state"])
        st = Guarded((N, H, S, S), init=d["state"])
        out = Guarded((N, T, H, S))
        ws = Guarded((gdn.gdn_prefill_workspace_bytes(N, T, HK, H, S),), dtype=torch.uint8)
        gdn.gdn_prefill_bf16(d["qkv"], d["z"], d["a"], d["b"], d["conv_w"], d["ssm_a"],
                             d["dt_bias"], d["norm_w"], cs.t, st.t, out.t, ws.t, HK, S ** -0.5,
                             scan=scan)
        for buf, name in ((cs, "conv_state"), (st, "state"), (out, "out"), (ws, "workspace")):
            buf.check(f"gdn_prefill_bf16 T={T} scan {scan} {name}")
