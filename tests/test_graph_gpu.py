"""The decode step captured in a HIP graph (needs an MI355X).

A caller that replays a captured decode step must get exactly what eager
launches give: the same kernels run on the same data. The step (conv, the
recurrence, the gated norm, and the fused bf16 layer) is captured once and
replayed several times, with eager work and synchronisation between the
replays, and every replay is compared with the eager result bit for bit. The
layer split over 64-row workgroups is captured too: its counters must be zero
again after every replay, since no replay clears them.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, dev, dev_ssm_a, upload_layer
from linear_attention_ssm_recurrence_amd import gdn, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def _bits(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


def test_decode_step_graph_replays_equal_eager():
    w = inputs.WORKLOADS[1]
    d = inputs.draw(w)
    H, HK, S = w.n_v_heads, w.n_k_heads, w.state_size
    q = torch.empty((1, H, S), device=DEV)
    k = torch.empty((1, H, S), device=DEV)
    g = torch.empty((1, H), device=DEV)
    beta = torch.empty((1, H), device=DEV)
    gdn.gdn_l2norm_gqa(dev(d["q_raw"][:, 0]), q, w.l2_eps)
    gdn.gdn_l2norm_gqa(dev(d["k_raw"][:, 0]), k, w.l2_eps)
    gdn.gdn_decay_gate(dev(d["a"][:, 0]), dev(d["dt_bias"]), dev_ssm_a(d["A_log"]), g)
    gdn.gdn_sigmoid(dev(d["b"][:, 0]), beta)
    v, z, x = dev(d["v"][:, 0]), dev(d["z"][:, 0]), dev(d["x"][:, 0])
    cw, nw = dev(d["conv_w"]), dev(d["norm_w"])
    wb = inputs.WORKLOADS[4]
    lb = inputs.draw_block_layer(0, wb, n_seqs=3)
    b_in = upload_layer(lb)
    ws = torch.zeros(gdn.gdn_decode_block_workspace_bytes(3, HK, H), dtype=torch.uint8,
                     device=DEV)

    def fresh():
        return {"st": dev(d["state"]), "cs": dev(d["conv_state"]),
                "bst": b_in["state"].clone(), "bcs": b_in["conv_state"].clone(),
                "y": torch.empty((1, H, S), device=DEV), "out": torch.empty((1, H, S), device=DEV),
                "co": torch.empty((1, w.conv_dim), device=DEV),
                "bout": torch.empty((3, H, S), device=DEV),
                "sst": b_in["state"].clone(), "scs": b_in["conv_state"].clone(),
                "sout": torch.empty((3, H, S), device=DEV)}

    def step(b):
        gdn.gdn_conv1d_silu(x, cw, b["cs"], b["co"])
        gdn.gdn_recurrence(b["st"], q, k, v, g, beta, b["y"], w.scale)
        gdn.gdn_gated_rmsnorm(b["y"], nw, z, b["out"], w.eps)
        gdn.gdn_decode_block_bf16(b_in["qkv"], b_in["z"], b_in["a"], b_in["b"], b_in["conv_w"],
                                  b_in["ssm_a"], b_in["dt_bias"], b_in["norm_w"], b["bcs"],
                                  b["bst"], b["bout"], HK, wb.scale, wb.l2_eps, wb.eps)
        gdn.gdn_decode_block_bf16_ex(b_in["qkv"], b_in["z"], b_in["a"], b_in["b"],
                                     b_in["conv_w"], b_in["ssm_a"], b_in["dt_bias"],
                                     b_in["norm_w"], b["scs"], b["sst"], b["sout"], ws, HK,
                                     wb.scale, wb.l2_eps, wb.eps)

    replays = 4
    eager = fresh()
    ref = []
    for _ in range(replays):
        step(eager)
        torch.cuda.synchronize()
        ref.append({key: val.clone() for key, val in eager.items()})

    cap = fresh()
    initial = {key: val.clone() for key, val in cap.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(fresh())                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cap)
    for key, val in initial.items():       # capture does not run the kernels; restore anyway
        cap[key].copy_(val)
    torch.cuda.synchronize()
    for r in range(replays):
        graph.replay()
        torch.cuda.synchronize()
        for key in ("st", "cs", "out", "co", "bst", "bcs", "bout", "sst", "scs", "sout"):
            assert torch.equal(cap[key], ref[r][key]), f"replay {r}: {key} differs from eager"
        assert int(ws.count_nonzero()) == 0, f"replay {r}: split-layer counters not zero"
        for a, b in (("sst", "bst"), ("scs", "bcs"), ("sout", "bout")):
            assert torch.equal(cap[a], cap[b]), f"replay {r}: split layer != one-workgroup layer"
        scratch = torch.randn(1 << 20, device=DEV)    # eager work between replays
        scratch.mul_(2.0)
        torch.cuda.synchronize()
