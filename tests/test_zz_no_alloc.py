"""The allocation-free split decode layer (gdn_decode_block_bf16_noalloc),
through the C ABI, against the workspace form (gdn_decode_block_bf16_ex) on
the same inputs, bit for bit (needs an MI355X).

Two calls in a row, the second with a smaller batch, each checked against
the workspace form; then the 64-sequence block workload, chained, and a
batch at the array's capacity. The library-owned counters are shared by
every call on the GPU, so each call depends on the previous one having left
them zero; the workspace form's own workspace is checked to be zero too.
"""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, dev, dev_bits, dev_ssm_a
from linear_attention_ssm_recurrence_amd import gdn, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


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


def _both(d, HK, steps=1):
    """steps chained calls of each form on its own copy of the layer's
    buffers; asserts bit equality after every call and a zero workspace."""
    N, H, S = d["z"].shape
    scale = 1.0 / math.sqrt(S)
    fixed = [dev(d["conv_w"]), dev_ssm_a(d["A_log"]), dev(d["dt_bias"]), dev(d["norm_w"])]
    act = [dev_bits(d["qkv"]), dev_bits(d["z"]), dev(d["a"]), dev(d["b"])]
    bufs = {form: {"conv_state": dev(d["conv_state"]), "state": dev(d["state"]),
                   "out": torch.empty((N, H, S), dtype=torch.float32, device=DEV)}
            for form in ("ws", "noalloc")}
    ws = torch.zeros(gdn.gdn_decode_block_workspace_bytes(N, HK, H), dtype=torch.uint8,
                     device=DEV)
    for t in range(steps):
        b = bufs["ws"]
        gdn.gdn_decode_block_bf16_ex(*act, *fixed, b["conv_state"], b["state"], b["out"], ws, HK,
                                     scale, 1e-6, 1e-6)
        b = bufs["noalloc"]
        gdn.gdn_decode_block_bf16_noalloc(*act, *fixed, b["conv_state"], b["state"], b["out"], HK,
                                          scale, 1e-6, 1e-6)
        torch.cuda.synchronize()
        for k in ("out", "state", "conv_state"):
            assert torch.equal(bufs["noalloc"][k], bufs["ws"][k]), \
                f"step {t}: allocation-free layer != workspace layer ({k} bits)"
        assert int(ws.count_nonzero()) == 0


def test_noalloc_two_calls_second_smaller():
    """A call at 24 sequences (16 -> 32 heads), then one at 5 sequences: the
    second reuses the counters the first left zero."""
    rng = np.random.default_rng(700)
    print("noalloc: 24 sequences, then 5", flush=True)
    _both(_rand_layer(rng, 24, 16, 2, 4), 16)
    _both(_rand_layer(rng, 5, 16, 2, 4), 16)


def test_noalloc_block_workload_chained():
    """Layer 3 of the 64-sequence block workload, three chained calls."""
    print("noalloc: block workload layer 3, 3 calls", flush=True)
    _both(inputs.draw_block_layer(3), inputs.WORKLOADS[4].n_k_heads, steps=3)


@pytest.mark.parametrize("GQ,K", [(1, 2), (4, 3)])
def test_noalloc_group_sizes(GQ, K):
    """Other group sizes and conv widths, with group counts that leave the
    grid's last row of eight groups part-empty (3 sequences x 3 K-heads)."""
    print(f"noalloc: GQ {GQ}, K {K}", flush=True)
    _both(_rand_layer(np.random.default_rng(710 + GQ), 3, 3, GQ, K), 3, steps=2)


def test_noalloc_at_capacity():
    """n_seqs * (HK + H) = the array's capacity exactly (1 K-head, 1 V-head,
    32768 sequences: a 2 GiB state, drawn on the device), against the
    workspace form; then one sequence more, which is refused with GDN_ESIZE
    before anything is launched."""
    print("noalloc: at capacity", flush=True)
    cap = gdn.GDN_NOALLOC_MAX_COUNTERS
    N, HK, H, S, K = cap // 2, 1, 1, 128, 4
    C = 2 * HK * S + H * S
    gen = torch.Generator(device=DEV).manual_seed(730)
    rn = lambda *shape, sd=1.0: torch.randn(shape, generator=gen, device=DEV) * sd
    bf = lambda x: (x.view(torch.int32) >> 16).to(torch.int16)   # truncated bf16 patterns
    act = [bf(rn(N, C)), bf(rn(N, H, S)), rn(N, H), rn(N, H)]
    fixed = [rn(C, K, sd=0.5), dev_ssm_a(rn(H)), rn(H, sd=0.1), 1 + rn(S, sd=0.1)]
    cs0, st0 = rn(N, C, K - 1), rn(N, H, S, S, sd=0.05)
    ws = torch.zeros(gdn.gdn_decode_block_workspace_bytes(N, HK, H), dtype=torch.uint8,
                     device=DEV)
    res = []
    for form in ("ws", "noalloc"):
        cs, st, out = cs0.clone(), st0.clone(), torch.empty((N, H, S), device=DEV)
        if form == "ws":
            gdn.gdn_decode_block_bf16_ex(*act, *fixed, cs, st, out, ws, HK, 0.1, 1e-6, 1e-6)
        else:
            gdn.gdn_decode_block_bf16_noalloc(*act, *fixed, cs, st, out, HK, 0.1, 1e-6, 1e-6)
        torch.cuda.synchronize()
        res.append((out, st, cs))
        del st
    for a, b in zip(*res):
        assert torch.equal(a, b)
    assert int(ws.count_nonzero()) == 0
    del res, st0
    N1 = N + 1
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_decode_block_bf16_noalloc(
            torch.zeros((N1, C), dtype=torch.int16, device=DEV),
            torch.zeros((N1, H, S), dtype=torch.int16, device=DEV),
            torch.zeros((N1, H), device=DEV), torch.zeros((N1, H), device=DEV), *fixed,
            torch.zeros((N1, C, K - 1), device=DEV), torch.zeros((N1, H, S, S), device=DEV),
            torch.zeros((N1, H, S), device=DEV), HK, 0.1)
    assert e.value.code == gdn.GDN_ESIZE


def test_noalloc_captured_graph_replays():
    """The allocation-free layer captured in a HIP graph (the callers it is
    for include code under capture), replayed four times with eager work and
    synchronisation between the replays: every replay equals eager calls of
    the workspace form, bit for bit, chained on the same buffers."""
    print("noalloc: graph capture", flush=True)
    rng = np.random.default_rng(740)
    d = _rand_layer(rng, 6, 16, 2, 4)
    N, H, S = d["z"].shape
    HK = 16
    scale = 1.0 / math.sqrt(S)
    fixed = [dev(d["conv_w"]), dev_ssm_a(d["A_log"]), dev(d["dt_bias"]), dev(d["norm_w"])]
    act = [dev_bits(d["qkv"]), dev_bits(d["z"]), dev(d["a"]), dev(d["b"])]

    def bufs():
        return {"cs": dev(d["conv_state"]), "st": dev(d["state"]),
                "out": torch.empty((N, H, S), dtype=torch.float32, device=DEV)}

    ws = torch.zeros(gdn.gdn_decode_block_workspace_bytes(N, HK, H), dtype=torch.uint8,
                     device=DEV)
    eager, ref = bufs(), []
    for _ in range(4):
        gdn.gdn_decode_block_bf16_ex(*act, *fixed, eager["cs"], eager["st"], eager["out"], ws,
                                     HK, scale, 1e-6, 1e-6)
        torch.cuda.synchronize()
        ref.append({k: v.clone() for k, v in eager.items()})

    cap = bufs()
    warm = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # a first call outside the capture
        gdn.gdn_decode_block_bf16_noalloc(*act, *fixed, warm["cs"], warm["st"], warm["out"], HK,
                                          scale, 1e-6, 1e-6)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.gdn_decode_block_bf16_noalloc(*act, *fixed, cap["cs"], cap["st"], cap["out"], HK,
                                          scale, 1e-6, 1e-6)
    torch.cuda.synchronize()
    for r in range(4):
        graph.replay()
        torch.cuda.synchronize()
        for k in ("out", "st", "cs"):
            assert torch.equal(cap[k], ref[r][k]), f"replay {r}: {k} differs from eager"
        scratch = torch.randn(1 << 20, device=DEV)    # eager work between replays
        scratch.mul_(2.0)
        torch.cuda.synchronize()
