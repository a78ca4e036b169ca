"""Every entry point enqueues on the stream the caller passes (needs an MI355X).

The decode, the scan and the fused layer are run on a side stream (with the
default stream busy on other work) and on the default stream; the results
must be identical bit for bit. The split decode layer also runs on two
streams at once, each call with its own workspace.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, dev, prep_recurrence, upload_layer
from linear_attention_ssm_recurrence_amd import gdn, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def _bits(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


def test_side_stream_equals_default_stream():
    w = inputs.WORKLOADS[0]
    d = inputs.draw(w)
    p = prep_recurrence(d, w)
    wb = inputs.WORKLOADS[4]
    lb = inputs.draw_block_layer(1, wb, n_seqs=4)
    H, HK, S = wb.n_v_heads, wb.n_k_heads, wb.state_size

    def run(stream):
        st_scan = dev(p["state"])
        y_scan = torch.empty(p["v"].shape, device=DEV)
        b_in = upload_layer(lb)
        out = torch.empty((4, H, S), device=DEV)
        with torch.cuda.stream(stream):
            gdn.gdn_recurrence_seq(st_scan, dev(p["q"]), dev(p["k"]), dev(p["v"]), dev(p["g"]),
                                   dev(p["beta"]), y_scan, w.scale)
            gdn.gdn_decode_block_bf16(b_in["qkv"], b_in["z"], b_in["a"], b_in["b"],
                                      b_in["conv_w"], b_in["ssm_a"], b_in["dt_bias"],
                                      b_in["norm_w"], b_in["conv_state"], b_in["state"], out, HK,
                                      wb.scale, wb.l2_eps, wb.eps)
        stream.synchronize()
        return st_scan, y_scan, b_in["state"], b_in["conv_state"], out

    torch.cuda.synchronize()
    ref = run(torch.cuda.current_stream())
    side = torch.cuda.Stream()
    busy = torch.randn(1 << 22, device=DEV)
    for _ in range(20):                       # keep the default stream busy meanwhile
        busy.mul_(1.0001)
    got = run(side)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_split_layer_on_two_streams_with_own_workspaces():
    """Two split decode layers in flight at once on two streams (different
    batches, each with its own workspace, as the header requires), repeated:
    each equals the one-workgroup layer on the same inputs, and both
    workspaces are zero afterwards."""
    wb = inputs.WORKLOADS[4]
    H, HK, S = wb.n_v_heads, wb.n_k_heads, wb.state_size
    layers = [inputs.draw_block_layer(l, wb, n_seqs=n) for l, n in ((2, 24), (3, 40))]

    def upload(lb):
        return upload_layer(lb)

    def call(fn, t, out, *extra):
        fn(t["qkv"], t["z"], t["a"], t["b"], t["conv_w"], t["ssm_a"], t["dt_bias"], t["norm_w"],
           t["conv_state"], t["state"], out, *extra, HK, wb.scale, wb.l2_eps, wb.eps)

    ref, got, wss = [], [], []
    for lb in layers:
        n = lb["a"].shape[0]
        r, g = upload(lb), upload(lb)
        ref.append((r, torch.empty((n, H, S), device=DEV)))
        got.append((g, torch.empty((n, H, S), device=DEV)))
        wss.append(torch.zeros(gdn.gdn_decode_block_workspace_bytes(n, HK, H), dtype=torch.uint8,
                               device=DEV))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(3):
        for (t, out) in ref:
            call(gdn.gdn_decode_block_bf16, t, out)
        for (t, out), ws, s in zip(got, wss, streams):
            with torch.cuda.stream(s):
                call(gdn.gdn_decode_block_bf16_ex, t, out, ws)
    torch.cuda.synchronize()
    for (r, ro), (g, go), ws in zip(ref, got, wss):
        assert torch.equal(ro, go)
        assert torch.equal(r["state"], g["state"])
        assert torch.equal(r["conv_state"], g["conv_state"])
        assert int(ws.count_nonzero()) == 0
