"""Helpers of the GPU parity tests: device transfer, oracle-side input
preparation and the tolerance check."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from linear_attention_ssm_recurrence_amd import inputs

# The parity bar: |gpu - ref| <= ATOL + RTOL * |ref| for every element
# (1e-4 relative / 1e-5 absolute; 2e-4 relative after a 4096-token scan).
RTOL, ATOL = 1e-4, 1e-5
RTOL_LONG_SCAN = 2e-4

DEV = torch.device("cuda:0")


def oracle_threads() -> int:
    n = min(16, os.cpu_count() or 1)
    oracle.set_threads(n)
    return n


def dev(x, dtype=np.float32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=dtype)).to(DEV)


def dev_bits(x) -> torch.Tensor:
    """uint16 bf16 bit patterns -> int16 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).to(DEV)


def dev_ssm_a(A_log) -> torch.Tensor:
    """The gate's per-head factor ssm_a = -exp(A_log) on the device, from the
    library's own kernel (gdn_ssm_a): the form every gate-forming entry point
    takes. A_log is a host array or a device tensor."""
    from linear_attention_ssm_recurrence_amd import gdn
    t = A_log if isinstance(A_log, torch.Tensor) else dev(A_log)
    out = torch.empty_like(t)
    gdn.gdn_ssm_a(t, out)
    torch.cuda.current_stream(out.device).synchronize()   # ready for any stream
    return out


def upload_layer(lb: dict) -> dict:
    """A fused-layer input dict on the device (bf16 patterns as int16), with
    ssm_a from the library beside A_log."""
    t = {key: (dev_bits(val) if val.dtype == np.uint16 else dev(val)) for key, val in lb.items()}
    t["ssm_a"] = dev_ssm_a(t["A_log"])
    return t


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def widen_bf16(t: torch.Tensor) -> torch.Tensor:
    """int16 bf16 patterns on the device -> float32 (exact), for staged paths."""
    return (t.to(torch.int32) << 16).view(torch.float32)


def assert_close(got, ref, what: str, rtol: float = RTOL, atol: float = ATOL) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite values in the GPU result"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err, -1)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
                             f"(rtol {rtol}, atol {atol}); worst at {i}: gpu {got[i]!r} "
                             f"ref {ref[i]!r}")
    return float(err.max()) if err.size else 0.0


def prep_recurrence(d: dict, w: inputs.Workload) -> dict:
    """Oracle-side preparation of the recurrence inputs from raw draws:
    L2 norm + tiled repeat of q and k, the decay gate and beta = sigmoid(b)."""
    return {
        "q": oracle.l2norm_gqa(d["q_raw"], w.n_v_heads, w.l2_eps),
        "k": oracle.l2norm_gqa(d["k_raw"], w.n_v_heads, w.l2_eps),
        "v": d["v"],
        "g": oracle.decay_gate(d["a"], d["dt_bias"], d["A_log"]),
        "beta": oracle.sigmoid(d["b"]),
        "state": d["state"],
    }
