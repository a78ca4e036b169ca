#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet hot path on one MI355X.

Headline (the JSON line's ``value``): decode state throughput of the gated
delta-rule recurrence for a batch of 256 independent sequences x 32 V-heads x
S = 128 (fp32 state, 512 MiB): state bytes read + written per launch (1 GiB)
divided by the time per launch. A step is one ``gdn_recurrence`` launch; the
benchmark alternates between two independent state buffers so that no step
finds its state in the 256 MB Infinity Cache.

The same line carries the other workloads of the hot path ("legs"):
  scan        1 sequence x 4096 tokens x 32 heads x S = 128: conv1d+SiLU over
              the 4096 x 8192 activations, then the chunked scan (the
              sequential scan timed beside it); tokens/s
  block       64 sequences x 48 layers of the fused bf16 decode layer (conv,
              L2 norm + GQA repeat 16 -> 32, gate, sigmoid, recurrence, gated
              RMSNorm), one launch per layer; ms per 48-layer step, for the
              layer split over 64-row workgroups (gdn_decode_block_bf16_ex)
              and, beside it, the one-workgroup-per-K-head layer
  decode_full the headline batch with its per-token glue launched too
              (decay gate, sigmoid, L2 norm + GQA of q and k) before the
              recurrence, and the same step as one launch (gdn_decode_step)
  decode_t4   the headline batch with the "T4" read-out (gdn_recurrence_ex)
  prefill     one bf16 layer over 1 sequence x 4096 positions through
              gdn_prefill_bf16_ex (fused conv/norm/gate front end, chunked scan
              with the 16 -> 32 repeat by index, gated norm; the sequential
              scan timed beside it); tokens/s
  spec        a speculative-decoding verify step: 64 sequences x 4 draft
              tokens, 16 -> 32 heads by index, S = 128, conv over C = 8192,
              with per-token state and conv snapshots
  single      one sequence, one token (16 -> 32 heads, S = 128, C = 8192):
              conv + recurrence + gated norm as three launches, and the fused
              bf16 layer as one; microseconds per step of GPU time with warm
              caches (a captured HIP graph replayed) and after a 1 GiB cache
              flush, and per eager Python call (host-launch-bound)
  machine     what this GPU achieves: a 1 GiB device copy (GB/s), the fp32
              FMA-chain issue rate of gdn_probe_fma (TFLOP/s), and the issue
              rate of fp32 and bf16 matrix instructions at one wave per SIMD
              (gdn_probe_mfma: cycles per instruction, TFLOP/s)
and the roofline of the dominant kernel (the decode recurrence) measured with
HIP events on the stream it runs on, and the CPU oracle timed on this host.

Inputs are seeded synthetic draws (numpy PCG64) with the workloads' shapes
and distributions, uploaded before timing; the per-token glue of the
recurrence inputs (q/k normalisation, gate, beta) runs on the GPU through the
library before the timed region.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs decode,scan,block]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN decode state GB/s (% HBM peak) @32h S=128; scan tokens/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor specification
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, vendor specification
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix, vendor specification


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--legs",
                    default="decode,scan,block,decode_full,decode_t4,spec,prefill,single,machine")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-runs", type=int, default=5,
                    help="timed runs of each oracle baseline (after one warm-up); the median "
                         "is reported")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy and a 512 MiB fill three times "
                         "each (known-size kernels for scaling hardware byte counters, and the "
                         "write-only rate)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

class Timer:
    """Wall clock bracketed by device synchronisation, plus HIP events on the
    current stream (the stream every library call here is enqueued on)."""

    def __init__(self, torch):
        self.torch = torch

    def __enter__(self):
        t = self.torch
        t.cuda.synchronize()
        self.ev0 = t.cuda.Event(enable_timing=True)
        self.ev1 = t.cuda.Event(enable_timing=True)
        self.w0 = time.perf_counter()
        self.ev0.record()
        return self

    def __exit__(self, *exc):
        self.ev1.record()
        self.torch.cuda.synchronize()
        self.wall_ms = (time.perf_counter() - self.w0) * 1e3
        self.event_ms = self.ev0.elapsed_time(self.ev1)
        return False


def parallel(fn, items, workers=16):
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


# ---------------------------------------------------------------------------
# legs
# ---------------------------------------------------------------------------

def dev_ssm_a(torch, gdn, A_log):
    """The gate's per-head factor ssm_a = -exp(A_log) on the device, prepared
    once per set of parameters by the library (gdn_ssm_a)."""
    src = torch.from_numpy(np.ascontiguousarray(A_log, dtype=np.float32)).cuda()
    out = torch.empty_like(src)
    gdn.gdn_ssm_a(src, out)
    return out


def decode_inputs(torch, gdn, inputs):
    w = inputs.WORKLOADS[2]
    d = inputs.draw(w)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    N, H, HK, S = w.n_seqs, w.n_v_heads, w.n_k_heads, w.state_size
    raw = {k: dev(d[k][:, 0]) for k in ("q_raw", "k_raw", "v", "a", "b")}
    par = {"ssm_a": dev_ssm_a(torch, gdn, d["A_log"]), "dt_bias": dev(d["dt_bias"])}
    q = torch.empty((N, H, S), device="cuda")
    k = torch.empty((N, H, S), device="cuda")
    g = torch.empty((N, H), device="cuda")
    beta = torch.empty((N, H), device="cuda")

    def glue():
        gdn.gdn_l2norm_gqa(raw["q_raw"], q, w.l2_eps)
        gdn.gdn_l2norm_gqa(raw["k_raw"], k, w.l2_eps)
        gdn.gdn_decay_gate(raw["a"], par["dt_bias"], par["ssm_a"], g)
        gdn.gdn_sigmoid(raw["b"], beta)

    glue()
    st0 = dev(d["state"])
    states = [st0, st0.clone()]
    y = torch.empty((N, H, S), device="cuda")
    torch.cuda.synchronize()
    return w, d, dict(q=q, k=k, v=raw["v"], g=g, beta=beta, y=y, states=states, glue=glue,
                      raw=raw, par=par)


def decode_bytes(w) -> dict:
    N, H, S = w.n_seqs, w.n_v_heads, w.state_size
    state = 2 * N * H * S * S * 4
    vecs = 4 * N * H * S * 4          # q, k, v read; y written
    scal = 2 * N * H * 4              # g, beta
    return {"state": state, "total": state + vecs + scal}


def run_decode(torch, gdn, inputs, steps, warmup, with_glue=False, t4=False, fused=False):
    w, d, t = decode_inputs(torch, gdn, inputs)

    def step(i):
        if fused:   # the glue folded into the recurrence kernel: one launch
            r, p = t["raw"], t["par"]
            gdn.gdn_decode_step(t["states"][i % 2], r["q_raw"], r["k_raw"], r["v"], r["a"], r["b"],
                                p["ssm_a"], p["dt_bias"], t["y"], w.scale, w.l2_eps)
            return
        if with_glue:
            t["glue"]()
        if t4:
            gdn.gdn_recurrence_ex(t["states"][i % 2], t["q"], t["k"], t["v"], t["g"], t["beta"],
                                  t["y"], w.scale, gdn.GDN_RECUR_T4)
        else:
            gdn.gdn_recurrence(t["states"][i % 2], t["q"], t["k"], t["v"], t["g"], t["beta"],
                               t["y"], w.scale)

    for i in range(warmup):
        step(i)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    with Timer(torch) as tm:
        for i in range(steps):
            if i:
                marks[i - 1].record()
            step(i)
        marks[-1].record()
    b = decode_bytes(w)
    ms_wall = tm.wall_ms / steps
    ms_ev = tm.event_ms / steps
    # per launch: from the previous launch's end mark (the timed region's start for
    # the first) to its own; the launches run back to back
    bounds = [tm.ev0] + marks
    per_launch = sorted(a.elapsed_time(c) for a, c in zip(bounds[:-1], bounds[1:]))
    res = {
        "workload": "batched decode: 256 sequences x 32 V-heads x S=128, fp32 state 512 MiB",
        "ms_per_step": ms_wall,
        "kernel_ms_events": ms_ev,
        "kernel_ms_median": per_launch[len(per_launch) // 2],
        "state_GBps": b["state"] / (ms_wall * 1e-3) / 1e9,
        "total_GBps": b["total"] / (ms_wall * 1e-3) / 1e9,
        "algorithmic_bytes_per_launch": b["total"],
        "state_bytes_per_launch": b["state"],
    }
    return w, d, res


def run_scan(torch, gdn, inputs, steps, warmup):
    w = inputs.WORKLOADS[3]
    d = inputs.draw(w)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    N, T, H, HK, S, C = w.n_seqs, w.n_tokens, w.n_v_heads, w.n_k_heads, w.state_size, w.conv_dim
    q = torch.empty((N, T, H, S), device="cuda")
    k = torch.empty((N, T, H, S), device="cuda")
    g = torch.empty((N, T, H), device="cuda")
    beta = torch.empty((N, T, H), device="cuda")
    gdn.gdn_l2norm_gqa(dev(d["q_raw"]), q, w.l2_eps)
    gdn.gdn_l2norm_gqa(dev(d["k_raw"]), k, w.l2_eps)
    gdn.gdn_decay_gate(dev(d["a"]), dev(d["dt_bias"]), dev_ssm_a(torch, gdn, d["A_log"]), g)
    gdn.gdn_sigmoid(dev(d["b"]), beta)
    v = dev(d["v"])
    st = dev(d["state"])
    y = torch.empty((N, T, H, S), device="cuda")
    x = dev(d["x"])
    cw = dev(d["conv_w"])
    cs = dev(d["conv_state"])
    co = torch.empty_like(x)
    torch.cuda.synchronize()

    def conv():
        gdn.gdn_conv1d_silu_seq(x, cw, cs, co)

    def scan():
        gdn.gdn_recurrence_seq(st, q, k, v, g, beta, y, w.scale)

    def scan_t4():   # the same scan with the "T4" read-out (same state, y regrouped)
        gdn.gdn_recurrence_seq_ex(st, q, k, v, g, beta, y, w.scale, variant=gdn.GDN_RECUR_T4)

    ws = torch.empty(gdn.gdn_chunked_workspace_bytes(N, T, H, S), dtype=torch.uint8, device="cuda")

    def chunked():
        gdn.gdn_recurrence_seq_chunked(st, q, k, v, g, beta, y, w.scale, ws)

    for _ in range(warmup):
        conv()
        chunked()
    with Timer(torch) as t_all:
        for _ in range(steps):
            conv()
            chunked()
    with Timer(torch) as t_all_seq:
        for _ in range(steps):
            conv()
            scan()
    # the conv alone over input/output sets in rotation (1 GiB in all, beyond
    # the 256 MB last-level cache), so that each launch reads its input from HBM
    xr = [x] + [x.clone() for _ in range(3)]
    orr = [co] + [torch.empty_like(co) for _ in range(3)]
    for i in range(4):
        gdn.gdn_conv1d_silu_seq(xr[i], cw, cs, orr[i])
    with Timer(torch) as t_conv:
        for i in range(steps):
            gdn.gdn_conv1d_silu_seq(xr[i % 4], cw, cs, orr[i % 4])
    with Timer(torch) as t_scan:
        for _ in range(steps):
            scan()
    with Timer(torch) as t_chunk:
        for _ in range(steps):
            chunked()
    scan_t4()
    with Timer(torch) as t_t4:
        for _ in range(steps):
            scan_t4()
    ms = t_all.wall_ms / steps
    scan_ms = t_scan.event_ms / steps
    conv_ms = t_conv.event_ms / steps
    flops = scan_method_flops(N, T, H, S)
    conv_bytes = 2 * N * T * C * 4 + C * w.conv_kernel * 4 + 2 * N * C * (w.conv_kernel - 1) * 4
    scan_bytes = (4 * N * T * H * S + 2 * N * T * H) * 4 + 2 * N * H * S * S * 4
    return {
        "workload": "scan: 1 sequence x 4096 tokens x 32 heads x S=128 fp32, chunked form, "
                    "preceded by conv1d+SiLU over 4096 x 8192 (K=4)",
        "ms_per_step": ms,
        "tokens_per_s": N * T / (ms * 1e-3),
        "sequential_ms_per_step": t_all_seq.wall_ms / steps,
        "scan_kernel_ms": scan_ms,
        "scan_tokens_per_s": N * T / (scan_ms * 1e-3),
        "scan_TFLOPs": flops / (scan_ms * 1e-3) / 1e12,
        "scan_frac_fp32_vector_peak": flops / (scan_ms * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
        "scan_algorithmic_bytes": scan_bytes,
        "scan_t4_kernel_ms": t_t4.event_ms / steps,
        "chunked_scan_ms": t_chunk.event_ms / steps,
        "chunked_scan_tokens_per_s": N * T / (t_chunk.event_ms / steps * 1e-3),
        "chunked_method_TFLOPs": flops / (t_chunk.event_ms / steps * 1e-3) / 1e12,
        "chunked_frac_method_flops": flops / (t_chunk.event_ms / steps * 1e-3) / 1e12
                                     / FP32_MFMA_PEAK_TFLOPS,
        "chunked_frac_method_flops_note": "the method's own 7 flop per state element and token "
                                          "over the fp32 matrix peak",
        "chunked_mfma_TFLOPs": chunked_mfma_flops(N, T, H, q.shape[2]) / (t_chunk.event_ms / steps * 1e-3) / 1e12,
        "chunked_mfma_pipe_frac": chunked_mfma_flops(N, T, H, q.shape[2]) / (t_chunk.event_ms / steps * 1e-3)
                                  / 1e12 / FP32_MFMA_PEAK_TFLOPS,
        "chunked_mfma_pipe_frac_note": "matrix-pipe utilisation: the MFMA work the chunked form "
                                       "executes (1.34x the method's flops: masked Gram tiles, "
                                       "the blockwise inverse) over the same peak",
        "conv_kernel_ms": conv_ms,
        "conv_note": "the conv alone, each launch on one of four input/output sets in rotation "
                     "(input cold in the last-level cache)",
        "conv_GBps": conv_bytes / (conv_ms * 1e-3) / 1e9,
        "conv_frac_hbm_peak": conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }


def w_scan_tokens(leg) -> float:
    """Tokens per step of the scan leg (conv + scan over one 4096-token sequence)."""
    return leg["tokens_per_s"] * leg["ms_per_step"] * 1e-3


def scan_method_flops(N, T, H, S) -> float:
    """The method's own arithmetic over a scan: per state element and token,
    the decay (1 mul) and three multiply-adds (the prediction, the rank-1
    update, the read-out), 7 flop; the same count for the sequential and
    the chunked form."""
    return 7.0 * N * T * H * S * S


def chunked_mfma_flops(N, T, H, HK=None) -> float:
    """fp32 MFMA work of one chunked scan at S = 128 (v_mfma_f32_16x16x4f32,
    2048 flop each): per 64-position chunk, the preparation runs 640 per
    K-head (20 Gram tiles x 32) and 64 per V-head (the blockwise inverse),
    and the scan's 8 row blocks x 4 waves run 128 each per V-head."""
    HK = H if HK is None else HK
    chunks = (T + 63) // 64
    return 2048.0 * N * chunks * (HK * 640 + H * (64 + 8 * 4 * 128))


def run_spec(torch, gdn, inputs, steps, warmup):
    """Verify step of speculative decoding: T draft tokens of N sequences
    through conv (with history snapshots) and the scan (with state
    snapshots), q/k repeated to the V-heads by index."""
    N, T, HK, H, S, C, K = 64, 4, 16, 32, 128, 8192, 4
    w = inputs.Workload(5, "spec", N, T, H, HK, S, conv_dim=C, state_sigma=0.05,
                        conv_state_sigma=1.0, seed=5)
    d = inputs.draw(w)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q = torch.empty((N, T, HK, S), device="cuda")
    k = torch.empty((N, T, HK, S), device="cuda")
    g = torch.empty((N, T, H), device="cuda")
    beta = torch.empty((N, T, H), device="cuda")
    gdn.gdn_l2norm_gqa(dev(d["q_raw"]), q, w.l2_eps)
    gdn.gdn_l2norm_gqa(dev(d["k_raw"]), k, w.l2_eps)
    gdn.gdn_decay_gate(dev(d["a"]), dev(d["dt_bias"]), dev_ssm_a(torch, gdn, d["A_log"]), g)
    gdn.gdn_sigmoid(dev(d["b"]), beta)
    v, st, x, cw, cs = (dev(d[key]) for key in ("v", "state", "x", "conv_w", "conv_state"))
    y = torch.empty((N, T, H, S), device="cuda")
    co = torch.empty_like(x)
    snaps = torch.empty((N, T, H, S, S), device="cuda")
    csnaps = torch.empty((N, T, C, K - 1), device="cuda")

    def step():
        gdn.gdn_conv1d_silu_seq_ex(x, cw, cs, co, csnaps)
        gdn.gdn_recurrence_seq_ex(st, q, k, v, g, beta, y, w.scale, snaps)

    for _ in range(warmup):
        step()
    with Timer(torch) as tm:
        for _ in range(steps):
            step()
    ms = tm.wall_ms / steps
    nbytes = (2 * N * H * S * S * 4 + N * T * H * S * S * 4      # state r+w, snapshots
              + 2 * N * T * HK * S * 4 + 2 * N * T * H * S * 4     # q, k; v, y
              + 2 * N * T * C * 4 + 2 * N * C * (K - 1) * 4 + N * T * C * (K - 1) * 4)
    return {"workload": "speculative verify: 64 sequences x 4 draft tokens, 16 -> 32 heads, "
                        "S=128, conv C=8192 K=4, state and history snapshots per token",
            "ms_per_step": ms, "tokens_per_s": N * T / (ms * 1e-3),
            "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def run_prefill(torch, gdn, inputs, steps, warmup):
    d = inputs.draw_prefill()
    N, T, H, S = d["z"].shape
    HK, K = 16, d["conv_w"].shape[1]

    def dev(x):
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()

    t = {key: dev(val) for key, val in d.items()}
    t["ssm_a"] = dev_ssm_a(torch, gdn, d["A_log"])
    out = torch.empty((N, T, H, S), device="cuda")
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(N, T, HK, H, S), dtype=torch.uint8,
                     device="cuda")
    scale = 1.0 / math.sqrt(S)
    torch.cuda.synchronize()

    def step(scan):
        gdn.gdn_prefill_bf16(t["qkv"], t["z"], t["a"], t["b"], t["conv_w"], t["ssm_a"],
                             t["dt_bias"], t["norm_w"], t["conv_state"], t["state"], out, ws, HK,
                             scale, scan=scan)

    ms = {}
    for scan in (gdn.GDN_SCAN_CHUNKED, gdn.GDN_SCAN_SEQUENTIAL):
        for _ in range(warmup):
            step(scan)
        with Timer(torch) as tm:
            for _ in range(steps):
                step(scan)
        ms[scan] = tm.wall_ms / steps
    chunk_ms, seq_ms = ms[gdn.GDN_SCAN_CHUNKED], ms[gdn.GDN_SCAN_SEQUENTIAL]
    return {"workload": "bf16 prefill of one layer: 1 sequence x 4096 positions, 16 -> 32 heads, "
                        "S=128, C=8192, K=4, chunked scan",
            "ms_per_step": chunk_ms, "tokens_per_s": N * T / (chunk_ms * 1e-3),
            "sequential_ms_per_step": seq_ms,
            "sequential_tokens_per_s": N * T / (seq_ms * 1e-3)}


def run_single(torch, gdn, inputs, steps, warmup):
    """One sequence, one token: latency of the decode kernels."""
    w = inputs.WORKLOADS[1]
    d = inputs.draw(w)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    H, HK, S, C, K = w.n_v_heads, w.n_k_heads, w.state_size, w.conv_dim, w.conv_kernel
    q = torch.empty((1, H, S), device="cuda")
    k = torch.empty((1, H, S), device="cuda")
    g = torch.empty((1, H), device="cuda")
    beta = torch.empty((1, H), device="cuda")
    gdn.gdn_l2norm_gqa(dev(d["q_raw"][:, 0]), q, w.l2_eps)
    gdn.gdn_l2norm_gqa(dev(d["k_raw"][:, 0]), k, w.l2_eps)
    gdn.gdn_decay_gate(dev(d["a"][:, 0]), dev(d["dt_bias"]), dev_ssm_a(torch, gdn, d["A_log"]), g)
    gdn.gdn_sigmoid(dev(d["b"][:, 0]), beta)
    v, st, z = dev(d["v"][:, 0]), dev(d["state"]), dev(d["z"][:, 0])
    x, cw, cs, nw = dev(d["x"][:, 0]), dev(d["conv_w"]), dev(d["conv_state"]), dev(d["norm_w"])
    y = torch.empty((1, H, S), device="cuda")
    out = torch.empty((1, H, S), device="cuda")
    co = torch.empty((1, C), device="cuda")
    # the fused bf16 layer on one sequence (layer 0 of the block workload's draws)
    wb = inputs.WORKLOADS[4]
    lb = inputs.draw_block_layer(0, wb, n_seqs=1)
    bits = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    b_in = {key: (bits(val) if val.dtype == np.uint16 else dev(val)) for key, val in lb.items()}
    b_in["ssm_a"] = dev_ssm_a(torch, gdn, lb["A_log"])
    b_out = torch.empty((1, H, S), device="cuda")
    flush = torch.empty(256 * 1024 * 1024, device="cuda")    # 1 GiB > the 256 MB Infinity Cache
    torch.cuda.synchronize()

    def three():
        gdn.gdn_conv1d_silu(x, cw, cs, co)
        gdn.gdn_recurrence(st, q, k, v, g, beta, y, w.scale)
        gdn.gdn_gated_rmsnorm(y, nw, z, out, w.eps)

    def fused():
        gdn.gdn_decode_block_bf16(b_in["qkv"], b_in["z"], b_in["a"], b_in["b"], b_in["conv_w"],
                                  b_in["ssm_a"], b_in["dt_bias"], b_in["norm_w"],
                                  b_in["conv_state"], b_in["state"], b_out, HK, wb.scale,
                                  wb.l2_eps, wb.eps)

    ws1 = torch.zeros(gdn.gdn_decode_block_workspace_bytes(1, HK, H), dtype=torch.uint8,
                      device="cuda")

    def fused_split():
        gdn.gdn_decode_block_bf16_ex(b_in["qkv"], b_in["z"], b_in["a"], b_in["b"],
                                     b_in["conv_w"], b_in["ssm_a"], b_in["dt_bias"],
                                     b_in["norm_w"], b_in["conv_state"], b_in["state"], b_out,
                                     ws1, HK, wb.scale, wb.l2_eps, wb.eps)

    def eager_us(fn):
        for _ in range(warmup):
            fn()
        with Timer(torch) as tm:
            for _ in range(steps):
                fn()
        return tm.event_ms / steps * 1e3

    def graph_us(fn, per_graph=20, replays=10):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                fn()
        graph.replay()
        with Timer(torch) as tm:
            for _ in range(replays):
                graph.replay()
        return tm.event_ms / (replays * per_graph) * 1e3

    def cold_us(fn, reps):
        evs = []
        for i in range(reps):
            flush.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)[reps // 2] * 1e3   # median

    reps = max(5, min(steps, 30))
    alg = (2 * H * S * S * 4 + 4 * H * S * 4 + 2 * H * 4           # recurrence
           + 2 * C * 4 + C * K * 4 + 2 * C * (K - 1) * 4           # conv
           + 3 * H * S * 4 + S * 4)                                # gated norm
    r = {"workload": "one sequence, one token: 16 -> 32 heads, S=128, C=8192, K=4",
         "three_kernels_us_warm": graph_us(three), "three_kernels_us_flushed": cold_us(three, reps),
         "three_kernels_us_eager": eager_us(three),
         "fused_bf16_layer_us_warm": graph_us(fused), "fused_bf16_layer_us_flushed": cold_us(fused, reps),
         "fused_bf16_layer_us_eager": eager_us(fused),
         "fused_bf16_layer_split_us_warm": graph_us(fused_split),
         "fused_bf16_layer_split_us_flushed": cold_us(fused_split, reps),
         "fused_bf16_layer_split_us_eager": eager_us(fused_split),
         "three_kernels_algorithmic_bytes": alg}
    r["three_kernels_GBps_flushed"] = alg / (r["three_kernels_us_flushed"] * 1e-6) / 1e9
    return r


def probe_fma_fn():
    """gdn_probe_fma from the benchmark's own probe library (built beside
    libgdn.so, not part of it)."""
    import ctypes
    path = os.path.join(ROOT, "linear_attention_ssm_recurrence_amd", "libgdn_probe.so")
    fn = ctypes.CDLL(path).gdn_probe_fma
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def probe_mfma_fn():
    """gdn_probe_mfma from the benchmark's probe library."""
    import ctypes
    path = os.path.join(ROOT, "linear_attention_ssm_recurrence_amd", "libgdn_probe.so")
    fn = ctypes.CDLL(path).gdn_probe_mfma
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def run_machine(torch, gdn, steps):
    """What this GPU achieves: a plain device copy and the fp32 FMA issue rate."""
    src = torch.ones(256 * 1024 * 1024, device="cuda")       # 1 GiB
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    reps = max(3, min(steps, 10))
    with Timer(torch) as tc:
        for _ in range(reps):
            dst.copy_(src)
    copy_gbps = 2 * src.numel() * 4 * reps / (tc.event_ms * 1e-3) / 1e9
    del src, dst
    blocks, iters = 256 * 8, 4096
    out = torch.empty(blocks * 256, device="cuda")
    probe = probe_fma_fn()
    stream = torch.cuda.current_stream().cuda_stream

    def fma():
        rc = probe(out.data_ptr(), blocks, iters, 0.999, 1e-3, stream)
        if rc != 0:
            raise RuntimeError(f"gdn_probe_fma returned {rc}")

    fma()
    with Timer(torch) as tf:
        for _ in range(reps):
            fma()
    flops = blocks * 256 * iters * 32 * reps
    res = {"copy_1GiB_GBps": copy_gbps, "copy_frac_hbm_peak": copy_gbps / HBM_PEAK_GBS,
           "fma_chain_TFLOPs": flops / (tf.event_ms * 1e-3) / 1e12,
           "fma_chain_frac_fp32_peak": flops / (tf.event_ms * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS}
    # matrix instructions at one wave per SIMD (256 workgroups of 4 waves): time per
    # instruction per wave, in cycles at the nominal 2.4 GHz
    mfma = probe_mfma_fn()
    miters = 2000
    for kind, name, fl in ((0, "f32_16x16x4", 2048), (1, "bf16_16x16x32", 16384)):
        for chains in (1, 2, 4):
            def run_m():
                rc = mfma(kind, chains, out.data_ptr(), 256, miters, stream)
                if rc != 0:
                    raise RuntimeError(f"gdn_probe_mfma returned {rc}")
            run_m()
            with Timer(torch) as tm:
                for _ in range(reps):
                    run_m()
            us = tm.event_ms * 1e3 / reps
            res[f"mfma_{name}_chains{chains}_cycles"] = us * 2400.0 / (miters * chains)
            res[f"mfma_{name}_chains{chains}_TFLOPs"] = 1024 * miters * chains * fl / (us * 1e-6) / 1e12
    return res


def block_layer_bytes(N, H, HK, S, K) -> int:
    C = 2 * HK * S + H * S
    return (2 * N * H * S * S * 4            # state read + write
            + 2 * N * C * (K - 1) * 4        # conv history read + write
            + N * C * 2 + N * H * S * 2      # qkv, z (bf16)
            + N * H * S * 4                  # out
            + C * K * 4 + 2 * N * H * 4 + 2 * H * 4 + S * 4)


def run_block(torch, gdn, inputs, steps, warmup):
    w = inputs.WORKLOADS[4]
    N, H, HK, S, K, Lyr = w.n_seqs, w.n_v_heads, w.n_k_heads, w.state_size, w.conv_kernel, w.layers
    layers = []

    def make(l):
        return inputs.draw_block_layer(l, w)

    for l0 in range(0, Lyr, 16):
        for l, d in zip(range(l0, min(Lyr, l0 + 16)), parallel(make, range(l0, min(Lyr, l0 + 16)))):
            dv = {}
            for key, val in d.items():
                arr = np.ascontiguousarray(val)
                if arr.dtype == np.uint16:
                    arr = arr.view(np.int16)
                dv[key] = torch.from_numpy(arr).cuda()
            dv["out"] = torch.empty((N, H, S), device="cuda")
            dv["ssm_a"] = dev_ssm_a(torch, gdn, d["A_log"])
            layers.append(dv)
        log(f"block: {len(layers)}/{Lyr} layers resident")
    torch.cuda.synchronize()

    ws = torch.zeros(gdn.gdn_decode_block_workspace_bytes(N, HK, H), dtype=torch.uint8,
                     device="cuda")

    def step_split():
        for t in layers:
            gdn.gdn_decode_block_bf16_ex(t["qkv"], t["z"], t["a"], t["b"], t["conv_w"],
                                         t["ssm_a"], t["dt_bias"], t["norm_w"], t["conv_state"],
                                         t["state"], t["out"], ws, HK, w.scale, w.l2_eps, w.eps)

    def step_one():
        for t in layers:
            gdn.gdn_decode_block_bf16(t["qkv"], t["z"], t["a"], t["b"], t["conv_w"], t["ssm_a"],
                                      t["dt_bias"], t["norm_w"], t["conv_state"], t["state"],
                                      t["out"], HK, w.scale, w.l2_eps, w.eps)

    times = {}
    for name, step in (("split", step_split), ("one", step_one)):
        for _ in range(warmup):
            step()
        with Timer(torch) as tm:
            for _ in range(steps):
                step()
        times[name] = tm.wall_ms / steps
    ms = times["split"]
    nbytes = Lyr * block_layer_bytes(N, H, HK, S, K)
    return {
        "workload": "fused bf16 decode layer: 64 sequences x 48 layers, 16 -> 32 heads, S=128, "
                    "C=8192, K=4, one launch per layer (gdn_decode_block_bf16_ex: 64-row "
                    "workgroups)",
        "ms_per_step": ms,
        "launches_per_step": Lyr,
        "GBps": nbytes / (ms * 1e-3) / 1e9,
        "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": nbytes,
        "one_workgroup_per_k_head_ms_per_step": times["one"],
        "one_workgroup_per_k_head_frac_hbm_peak":
            nbytes / (times["one"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }


DECODE_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "recurrence_decode_256x32x128_traffic.md")
DECODE_SOURCES = ("linear_attention_ssm_recurrence_amd/csrc/gdn_decode.hpp",
                  "linear_attention_ssm_recurrence_amd/csrc/gdn_device.hpp")


def recorded_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None
    when the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        text = open(DECODE_TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256", "").strip() != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def _median_seconds(run, runs):
    """Median wall time of `runs` calls of run() after one untimed warm-up."""
    run()
    times = []
    for _ in range(max(1, runs)):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    return float(np.median(times))


def cpu_baseline(inputs, d, runs):
    """The C oracle timed on this host's cores, in the GPU legs' units, each
    figure the median of `runs` timed runs after a warm-up, on all host
    threads (OpenMP over independent rows) and on one:
      decode  the headline batch, all 256 sequences (512 MiB of state, far
              beyond the host's caches): state GB/s, 10 steps per run on all
              threads, one step per run on one thread;
      scan    the scan workload (one sequence, 32 heads, S = 128) over its
              first 512 of 4096 tokens (a scan's cost per token is the same at
              every position): tokens/s;
      block   the fused bf16 layer on 64 sequences, two distinct layers of the
              48-layer workload per run: ms per 48-layer step (48 x the
              median time per layer).
    The oracle routines are called directly on arrays prepared once (the
    test front end's defensive copies are not timed)."""
    import ctypes
    import oracle
    threads = host_threads()
    lib = oracle._lib("f32")
    f32 = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    out = {}

    def both(name, make_run, per_run_multi, per_run_single):
        res = {}
        for label, nthreads, per_run in (("all", threads, per_run_multi),
                                         ("one", 1, per_run_single)):
            oracle.set_threads(nthreads)
            res[label] = (_median_seconds(make_run(per_run), runs), per_run)
        oracle.set_threads(threads)
        log(f"cpu baseline {name}: {res}")
        return res

    # decode: all 256 sequences of the headline batch
    w = inputs.WORKLOADS[2]
    n, H, S = w.n_seqs, w.n_v_heads, w.state_size
    q = f32(oracle.l2norm_gqa(d["q_raw"], H, w.l2_eps))
    k = f32(oracle.l2norm_gqa(d["k_raw"], H, w.l2_eps))
    g = f32(oracle.decay_gate(d["a"], d["dt_bias"], d["A_log"]))
    beta = f32(oracle.sigmoid(d["b"]))
    v = f32(d["v"])
    st = f32(d["state"]).copy()
    y = np.empty_like(v)

    def decode_run(steps):
        def run():
            for _ in range(steps):
                lib.oracle_recurrence_seq(P(st), P(q), P(k), P(v), P(g), P(beta), P(y), n, 1, H,
                                          S, float(w.scale))
        return run

    r = both("decode", decode_run, 10, 1)
    state_bytes = 2 * n * H * S * S * 4
    dec = {lab: state_bytes * steps / sec / 1e9 for lab, (sec, steps) in r.items()}
    del q, k, v, st, y

    # scan: the first 512 tokens of the scan workload, all 32 heads
    ws = inputs.WORKLOADS[3]
    dsc = inputs.draw(ws)
    Tn = 512
    Hs, Ss = ws.n_v_heads, ws.state_size
    sq = f32(oracle.l2norm_gqa(dsc["q_raw"][:, :Tn], Hs, ws.l2_eps))
    sk = f32(oracle.l2norm_gqa(dsc["k_raw"][:, :Tn], Hs, ws.l2_eps))
    sg = f32(oracle.decay_gate(dsc["a"][:, :Tn], dsc["dt_bias"], dsc["A_log"]))
    sb = f32(oracle.sigmoid(dsc["b"][:, :Tn]))
    sv = f32(dsc["v"][:, :Tn])
    sy = np.empty_like(sv)
    s0 = f32(dsc["state"])
    sst = s0.copy()

    def scan_run(_):
        def run():
            sst[...] = s0
            lib.oracle_recurrence_seq(P(sst), P(sq), P(sk), P(sv), P(sg), P(sb), P(sy), 1, Tn, Hs,
                                      Ss, float(ws.scale))
        return run

    r = both("scan", scan_run, 1, 1)
    scan = {lab: Tn / sec for lab, (sec, _) in r.items()}
    del dsc, sq, sk, sv, sy

    # block: two layers of the 64-sequence, 48-layer bf16 workload
    wb = inputs.WORKLOADS[4]
    layers = []
    for l in (0, 1):
        lb = inputs.draw_block_layer(l, wb)
        t = {key: (np.ascontiguousarray(val) if val.dtype == np.uint16 else f32(val))
             for key, val in lb.items()}
        t["out"] = np.empty((wb.n_seqs, wb.n_v_heads, wb.state_size), dtype=np.float32)
        layers.append(t)

    def block_run(_):
        def run():
            for t in layers:
                lib.oracle_decode_block_bf16(
                    P(t["qkv"]), P(t["z"]), P(t["a"]), P(t["b"]), P(t["conv_w"]), P(t["A_log"]),
                    P(t["dt_bias"]), P(t["norm_w"]), P(t["conv_state"]), P(t["state"]),
                    P(t["out"]), wb.n_seqs, wb.n_k_heads, wb.n_v_heads, wb.state_size,
                    wb.conv_kernel, float(wb.scale), float(wb.l2_eps), float(wb.eps))
        return run

    r = both("block", block_run, 1, 1)
    block = {lab: sec / len(layers) * wb.layers * 1e3 for lab, (sec, _) in r.items()}
    out = {"value": dec["all"], "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": (f"the decode step of all 256 sequences (all 32 V-heads, S=128, 512 MiB "
                      f"of state): state bytes read+written per second, median of {runs} runs "
                      f"of 10 steps after a warm-up, on {threads} threads"),
           "single_thread_value": dec["one"],
           "single_thread_sample": f"the same, one step per run, on 1 thread",
           "scan": {"value": scan["all"], "unit": "tokens/s", "cores": threads,
                    "single_thread_value": scan["one"],
                    "sample": (f"the sequential scan over the first {Tn} of the 4096 tokens of "
                               f"the scan workload (1 sequence, 32 heads, S=128, from a zero "
                               f"state), median of {runs} runs after a warm-up")},
           "block": {"value": block["all"], "unit": "ms per 48-layer step", "cores": threads,
                     "single_thread_value": block["one"],
                     "sample": (f"the fused bf16 decode layer on 64 sequences (16 -> 32 heads, "
                                f"S=128, C=8192, K=4), layers 0 and 1 of the workload per run; "
                                f"48 x the median time per layer over {runs} runs after a "
                                f"warm-up")}}
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the gated delta-rule path shards by sequence and "
              "head with no exchange, and the benchmark measures one GPU's share (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_ssm_recurrence_amd import gdn, inputs
    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    gdn.load_library()
    legs = [s.strip() for s in args.legs.split(",") if s.strip()]
    K, W = args.steps, args.warmup

    log("leg decode: 256 x 32 x 128 recurrence")
    w, d, dec = run_decode(torch, gdn, inputs, K, W)
    torch.cuda.empty_cache()
    out_legs = {}
    if "decode_full" in legs:
        log("leg decode_full")
        _, _, full = run_decode(torch, gdn, inputs, K, W, with_glue=True)
        _, _, fused = run_decode(torch, gdn, inputs, K, W, fused=True)
        out_legs["decode_full"] = {"ms_per_step": full["ms_per_step"],
                                   "state_GBps": full["state_GBps"],
                                   "fused_step_ms_per_step": fused["ms_per_step"],
                                   "fused_step_state_GBps": fused["state_GBps"]}
        torch.cuda.empty_cache()
    if "decode_t4" in legs:
        log("leg decode_t4")
        _, _, t4 = run_decode(torch, gdn, inputs, K, W, t4=True)
        out_legs["decode_t4"] = {"ms_per_step": t4["ms_per_step"], "state_GBps": t4["state_GBps"]}
        torch.cuda.empty_cache()
    if "spec" in legs:
        log("leg spec: 64 seqs x 4 draft tokens with snapshots")
        out_legs["spec"] = run_spec(torch, gdn, inputs, K, W)
        torch.cuda.empty_cache()
    if "prefill" in legs:
        log("leg prefill: bf16 layer, 4096 positions")
        out_legs["prefill"] = run_prefill(torch, gdn, inputs, K, W)
        torch.cuda.empty_cache()
    if "scan" in legs:
        log("leg scan: conv 4096x8192 + recurrence T=4096")
        out_legs["scan"] = run_scan(torch, gdn, inputs, K, W)
        torch.cuda.empty_cache()
    if "block" in legs:
        log("leg block: 64 seqs x 48 layers")
        out_legs["block"] = run_block(torch, gdn, inputs, K, W)
        torch.cuda.empty_cache()
    if "single" in legs:
        log("leg single: one sequence, one token")
        out_legs["single"] = run_single(torch, gdn, inputs, K, W)
        torch.cuda.empty_cache()
    if "machine" in legs:
        log("leg machine: device copy and FMA-chain rate")
        out_legs["machine"] = run_machine(torch, gdn, K)
        torch.cuda.empty_cache()

    if args.calibrate_copy:
        log("copy calibration: 3 x 512 MiB device-to-device copy, 3 x 512 MiB fill")
        src = torch.ones(128 * 1024 * 1024, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        with Timer(torch) as tc:
            for _ in range(3):
                dst.copy_(src)
        for _ in range(3):
            dst.fill_(1.0)
        with Timer(torch) as tf:
            for _ in range(3):
                dst.fill_(1.0)
        line_copy = {"bytes_read_per_copy": src.numel() * 4, "bytes_written_per_copy": src.numel() * 4,
                     "GBps": 2 * src.numel() * 4 * 3 / (tc.event_ms * 1e-3) / 1e9,
                     "fill_bytes_written": dst.numel() * 4,
                     "fill_GBps": dst.numel() * 4 * 3 / (tf.event_ms * 1e-3) / 1e9}
        del src, dst
    achieved = dec["algorithmic_bytes_per_launch"] / (dec["kernel_ms_events"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": dec["state_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded numpy PCG64 draws with the workloads' shapes and "
                "distributions; no dataset, no trained weights",
        "config": {"workload": dec["workload"], "n_seqs": w.n_seqs, "n_v_heads": w.n_v_heads,
                   "n_k_heads": w.n_k_heads, "state_size": w.state_size,
                   "state_bytes_per_step": dec["state_bytes_per_launch"]},
        "frac_hbm_peak_state": dec["state_GBps"] / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": "recurrence_decode_kernel<128,8>",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "kernel_ms": dec["kernel_ms_events"],
                     "kernel_ms_median": dec["kernel_ms_median"],
                     "bytes_per_launch": dec["algorithmic_bytes_per_launch"],
                     "traffic": recorded_traffic()},
        "legs": out_legs,
    }
    if args.calibrate_copy:
        line["copy_calibration"] = line_copy
    if "scan" in out_legs:
        line["scan_tokens_per_s"] = out_legs["scan"]["tokens_per_s"]
        line["scan_tokens_per_s_note"] = ("conv1d+SiLU then the chunked scan; the sequential scan "
                                          "(VALU) is scan_sequential_tokens_per_s")
        line["scan_sequential_tokens_per_s"] = (
            w_scan_tokens(out_legs["scan"]) / (out_legs["scan"]["sequential_ms_per_step"] * 1e-3))
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {host_threads()} threads and on 1")
        line["cpu_baseline"] = cpu_baseline(inputs, d, args.cpu_runs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
