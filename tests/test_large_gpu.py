"""Maximum sizes: every entry point family at a size whose flattened element
count passes 2^31, so that an offset computed in 32 bits anywhere would land
in the wrong place (needs an MI355X; about 30 GB of device memory).

The inputs are seeded synthetic draws made on the device (torch's CUDA
generator: at these sizes a host draw would take minutes), with the shapes
and distributions of the workloads. The oracle sees only sampled slices,
read back before the library call:
- decode, the fused layer: sampled (sequence, head) pairs, each on its own
  (the pairs are independent);
- the conv scan: sampled channels over the last positions (an output depends
  only on the K-1 inputs before it);
- the gated norm: sampled rows;
- the scans: with beta = 1 and each token's k a unit vector e_i whose index
  runs through all S columns every S consecutive tokens, a token sets column
  i of every state row to its v and leaves the other columns decayed, so the
  state after any S consecutive tokens no longer depends on where they
  started. The oracle run over the last 2S tokens from a zero state
  therefore gives the y of the last S tokens and the final state exactly
  (up to rounding), at offsets past 2^31.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, assert_close, dev_ssm_a, host, oracle_threads
from linear_attention_ssm_recurrence_amd import gdn

pytestmark = pytest.mark.gpu
TWO31 = 1 << 31


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < 40 * (1 << 30):
        pytest.skip("needs about 40 GB of free device memory")
    gdn.load_library()
    oracle_threads()
    yield
    torch.cuda.empty_cache()


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _randn(shape, gen, scale=1.0):
    return torch.randn(shape, device=DEV, generator=gen) * scale


def _unit(shape, gen):
    return torch.nn.functional.normalize(_randn(shape, gen), dim=-1)


def test_decode_state_past_2g_elements():
    N, HK, H, S = 4097, 16, 32, 128
    assert N * H * S * S > TWO31
    gen = _gen(51)
    state = _randn((N, H, S, S), gen, 0.05)
    qh, kh = _unit((N, HK, S), gen), _unit((N, HK, S), gen)
    v = _randn((N, H, S), gen)
    g = -torch.rand((N, H), device=DEV, generator=gen) * 0.5
    beta = torch.rand((N, H), device=DEV, generator=gen)
    pairs = [(0, 0), (2048, 17), (N - 1, 2), (N - 1, H - 1)]
    st0 = {pr: host(state[pr]) for pr in pairs}
    y = torch.empty((N, H, S), device=DEV)
    scale = 1 / math.sqrt(S)
    gdn.gdn_recurrence_ex(state, qh, kh, v, g, beta, y, scale, gdn.GDN_RECUR_EXACT)
    for n, h in pairs:
        one = lambda t: host(t[n, h % HK])[None, None]
        y_ref, st_ref = oracle.recurrence(st0[(n, h)][None, None], one(qh), one(kh),
                                          host(v[n, h])[None, None], host(g[n, h]).reshape(1, 1),
                                          host(beta[n, h]).reshape(1, 1), scale)
        assert_close(host(y[n, h]), y_ref[0, 0], f"decode y ({n}, {h})")
        assert_close(host(state[n, h]), st_ref[0, 0], f"decode state ({n}, {h})")


def test_decode_step_state_past_2g_elements():
    """The one-launch decode step from raw inputs, state past 2^31 elements."""
    N, HK, H, S = 4097, 16, 32, 128
    assert N * H * S * S > TWO31
    gen = _gen(56)
    state = _randn((N, H, S, S), gen, 0.05)
    q, k = _randn((N, HK, S), gen), _randn((N, HK, S), gen)
    v = _randn((N, H, S), gen)
    a, b = _randn((N, H), gen), _randn((N, H), gen)
    A_log, dt_bias = _randn((H,), gen), _randn((H,), gen, 0.5)
    pairs = [(0, 0), (2048, 17), (N - 1, 2), (N - 1, H - 1)]
    st0 = {pr: host(state[pr]) for pr in pairs}
    y = torch.empty((N, H, S), device=DEV)
    scale = 1 / math.sqrt(S)
    gdn.gdn_decode_step(state, q, k, v, a, b, dev_ssm_a(A_log), dt_bias, y, scale)
    g_ref = oracle.decay_gate(host(a), host(dt_bias), host(A_log))
    b_ref = oracle.sigmoid(host(b))
    for n, h in pairs:
        unit = lambda t: oracle.l2norm_gqa(host(t[n, h % HK])[None, None], 1)
        y_ref, st_ref = oracle.recurrence(st0[(n, h)][None, None], unit(q), unit(k),
                                          host(v[n, h])[None, None], g_ref[n, h].reshape(1, 1),
                                          b_ref[n, h].reshape(1, 1), scale)
        assert_close(host(y[n, h]), y_ref[0, 0], f"decode step y ({n}, {h})")
        assert_close(host(state[n, h]), st_ref[0, 0], f"decode step state ({n}, {h})")


@pytest.mark.parametrize("path", ["sequential", "chunked"])
def test_scan_tokens_past_2g_elements(path):
    N, T, HK, H, S = 2, 270_000, 1, 32, 128
    assert N * T * H * S > TWO31
    gen = _gen(52)
    q = _unit((N, T, HK, S), gen)
    k = torch.zeros((N, T, HK, S), device=DEV)
    t_idx = torch.arange(T, device=DEV)
    for n in range(N):
        k[n, t_idx, 0, (5 * t_idx + 3 * n) % S] = 1.0     # every S consecutive tokens: all columns
    v = _randn((N, T, H, S), gen)
    g = -torch.rand((N, T, H), device=DEV, generator=gen) * 0.3
    beta = torch.ones((N, T, H), device=DEV)
    state = _randn((N, H, S, S), gen, 0.05)
    W = 2 * S
    heads = [0, 5, H - 1]
    # oracle inputs of the sampled windows, read before the call
    win = {}
    for n, a in ((N - 1, T - W), (0, T - W), (N - 1, 0)):
        sl = lambda x: host(x[n, a:a + W])
        win[(n, a)] = dict(q=np.repeat(sl(q), len(heads), axis=1), k=np.repeat(sl(k), len(heads), axis=1),
                           v=sl(v)[:, heads], g=sl(g)[:, heads], beta=sl(beta)[:, heads])
    st_first = host(state[N - 1])[heads]
    y = torch.empty((N, T, H, S), device=DEV)
    scale = 1 / math.sqrt(S)
    if path == "sequential":
        gdn.gdn_recurrence_seq_ex(state, q, k, v, g, beta, y, scale)
    else:
        ws = torch.empty(gdn.gdn_chunked_workspace_bytes(N, T, H, S), dtype=torch.uint8, device=DEV)
        gdn.gdn_recurrence_seq_chunked(state, q, k, v, g, beta, y, scale, ws)
        del ws
    assert (N - 1) * T * H * S + (T - W) * H * S > TWO31        # the last window lies past 2^31
    for (n, a), w in win.items():
        start = st_first[None] if a == 0 else np.zeros((1, len(heads), S, S), np.float32)
        y_ref, st_ref = oracle.recurrence_seq(start, w["q"][None], w["k"][None], w["v"][None],
                                              w["g"][None], w["beta"][None], scale)
        got = host(y[n, a:a + W])[:, heads]
        first = 0 if a == 0 else S       # from a zero start, the first S outputs are not determined
        assert_close(got[first:], y_ref[0, first:], f"{path} scan y, seq {n}, tokens {a}+")
        if a + W == T:
            assert_close(host(state[n])[heads], st_ref[0], f"{path} scan final state, seq {n}")


def test_conv_scan_past_2g_elements():
    N, T, C, K = 1, 270_000, 8192, 4
    assert N * T * C > TWO31
    gen = _gen(53)
    x = _randn((N, T, C), gen)
    w = _randn((C, K), gen, 0.5)
    cs = _randn((N, C, K - 1), gen)
    chans = [0, 4097, C - 1]
    L = 64
    x_win = host(x[:, T - L:, chans])
    hist_before = np.ascontiguousarray(host(x[0, T - L - (K - 1):T - L, chans]).T[None])
    out = torch.empty((N, T, C), device=DEV)
    gdn.gdn_conv1d_silu_seq(x, w, cs, out)
    out_ref, cs_ref = oracle.conv1d_silu_seq(x_win, host(w[chans]), hist_before)
    assert_close(host(out[:, T - L:, chans]), out_ref, "conv out, last positions")
    assert np.array_equal(host(cs[:, chans]), cs_ref), "conv history after the last position"


def test_gated_norm_rows_past_2g_elements():
    D = 128
    rows = TWO31 // D + 64
    gen = _gen(54)
    y = _randn((rows, D), gen)
    z = _randn((rows, D), gen)
    w = 1 + _randn((D,), gen, 0.1)
    pick = [0, rows // 2, rows - 65, rows - 1]
    y_s, z_s = host(y[pick]), host(z[pick])
    out = torch.empty((rows, D), device=DEV)
    gdn.gdn_gated_rmsnorm(y, w, z, out, 1e-6)
    assert_close(host(out[pick]), oracle.gated_rmsnorm(y_s, host(w), z_s), "gated norm rows")


@pytest.mark.parametrize("split", [False, True], ids=["one_workgroup", "split_64_rows"])
def test_decode_block_state_past_2g_elements(split):
    N, HK, H, S, K = 4100, 16, 32, 128, 4
    C = 2 * HK * S + H * S
    assert N * H * S * S > TWO31
    gen = _gen(55)
    bits = lambda shape: _randn(shape, gen).to(torch.bfloat16).view(torch.int16)
    qkv, z = bits((N, C)), bits((N, H, S))
    a, b = _randn((N, H), gen), _randn((N, H), gen)
    conv_w = _randn((C, K), gen, 0.5)
    A_log, dt_bias = _randn((H,), gen), torch.zeros(H, device=DEV)
    ssm_a = dev_ssm_a(A_log)
    norm_w = 1 + _randn((S,), gen, 0.1)
    conv_state = _randn((N, C, K - 1), gen)
    state = _randn((N, H, S, S), gen, 0.05)
    seqs = [0, N - 1]
    before = {n: dict(qkv=host(qkv[n:n + 1]).view(np.uint16), z=host(z[n:n + 1]).view(np.uint16),
                      a=host(a[n:n + 1]), b=host(b[n:n + 1]), cs=host(conv_state[n:n + 1]),
                      st=host(state[n:n + 1])) for n in seqs}
    out = torch.empty((N, H, S), device=DEV)
    scale = 1 / math.sqrt(S)
    if split:
        ws = torch.zeros(gdn.gdn_decode_block_workspace_bytes(N, HK, H), dtype=torch.uint8,
                         device=DEV)
        gdn.gdn_decode_block_bf16_ex(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state,
                                     state, out, ws, HK, scale)
        assert int(ws.count_nonzero()) == 0, "split layer: workspace not zero after the call"
    else:
        gdn.gdn_decode_block_bf16(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state,
                                  state, out, HK, scale)
    for n in seqs:
        d = before[n]
        o_ref, cs_ref, st_ref = oracle.decode_block_bf16(
            d["qkv"], d["z"], d["a"], d["b"], host(conv_w), host(A_log), host(dt_bias),
            host(norm_w), d["cs"], d["st"], HK, scale)
        assert_close(host(out[n:n + 1]), o_ref, f"block out, seq {n}")
        assert_close(host(state[n:n + 1]), st_ref, f"block state, seq {n}")
        assert np.array_equal(host(conv_state[n:n + 1]), cs_ref), f"block history, seq {n}"
