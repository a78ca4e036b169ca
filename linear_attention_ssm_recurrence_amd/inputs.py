"""Seeded synthetic inputs for the Gated DeltaNet block.

This module only draws random numbers. It holds none of the block's arithmetic:
the L2 normalisation of q and k, the sigmoid of b and the decay gate are
computed by whoever consumes these draws (the HIP library on the product path,
the oracle in the tests).

Recipe. Each array comes from ``numpy.random.default_rng(seed)`` (PCG64) as
``standard_normal(shape, dtype=float32)`` scaled by sigma (and shifted where
stated), drawn in this fixed order:

    q, k, v, a, b, A_log, state, conv_w, conv_state, x, norm_w, z

An array a config does not use is not drawn, so it consumes no randomness.
bf16 arrays (the block workload) are the float32 draws rounded to bf16 with
round-to-nearest-even and carried as uint16 bit patterns.

Workloads (H V-heads, HK K-heads, S state size, T tokens, N sequences):

    0  tiny oracle check   N=1   T=8    H=HK=2  S=32            state 0
    1  single decode       N=1   T=1    H=32 HK=16 S=128  conv C=8192 K=4
    2  batched decode      N=256 T=1    H=32 HK=16 S=128        state N(0,.05)
    3  sequential scan     N=1   T=4096 H=HK=32 S=128          state 0
                           + conv stage x [4096][8192], zero history
    4  decode block, bf16  N=64  48 layers, H=32 HK=16 S=128 C=8192 K=4,
                           layer l drawn from seed 4000 + l

draw_prefill() draws one layer of a bf16 prefill over T positions with the
decode block's distributions (the default seed and sizes: 1 sequence, 4096
positions, 16 -> 32 heads, S=128, C=8192, K=4, zero initial state and history).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    n_seqs: int
    n_tokens: int
    n_v_heads: int
    n_k_heads: int
    state_size: int
    conv_dim: int = 0
    conv_kernel: int = 4
    state_sigma: float = 0.0      # 0 means a zero initial state
    conv_state_sigma: float = 0.0  # 0 means a zero initial history
    layers: int = 1
    seed: int = 0
    eps: float = 1e-6
    l2_eps: float = 1e-6
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.state_size))


WORKLOADS = {
    0: Workload(0, "tiny: 1 seq, 2 heads, S=32, T=8", 1, 8, 2, 2, 32, seed=0),
    1: Workload(1, "single decode: 1 seq, 32 V-heads (16 K-heads), S=128", 1, 1, 32, 16, 128,
                conv_dim=8192, state_sigma=0.05, conv_state_sigma=1.0, seed=1),
    2: Workload(2, "batched decode: 256 seqs, 32 V-heads (16 K-heads), S=128", 256, 1, 32, 16,
                128, state_sigma=0.05, seed=2),
    3: Workload(3, "sequential scan: 1 seq, T=4096, 32 heads, S=128", 1, 4096, 32, 32, 128,
                conv_dim=8192, seed=3),
    4: Workload(4, "decode block bf16: 64 seqs x 48 layers, 32 V-heads (16 K-heads), S=128",
                64, 1, 32, 16, 128, conv_dim=8192, state_sigma=0.05, conv_state_sigma=1.0,
                layers=48, seed=4000),
}


def normal(rng: np.random.Generator, shape, sigma: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 N(mean, sigma^2) draws (sigma is the standard deviation)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(w: Workload | int, seed: int | None = None, n_seqs: int | None = None,
         n_tokens: int | None = None, with_conv: bool | None = None) -> dict:
    """Raw draws for a recurrence/companion workload (configs 0-3).

    Returns float32 arrays:
      q_raw, k_raw [N][T][HK][S]   (to be L2-normalised and repeated to H heads)
      v            [N][T][H][S]
      a, b         [N][T][H]       (gate pre-activation, beta pre-sigmoid)
      A_log        [H]; dt_bias [H] (zeros)
      state        [N][H][S][S]    (transposed layout; zeros when sigma is 0)
      conv_w [C][K], conv_state [N][C][K-1], x [N][T][C]   (when with_conv)
      norm_w [S], z [N][T][H][S]
    Sizes can be overridden (``n_seqs``/``n_tokens``) for small parity cases.
    """
    if isinstance(w, int):
        w = WORKLOADS[w]
    N = w.n_seqs if n_seqs is None else n_seqs
    T = w.n_tokens if n_tokens is None else n_tokens
    H, HK, S = w.n_v_heads, w.n_k_heads, w.state_size
    conv = (w.conv_dim > 0) if with_conv is None else with_conv
    C = w.conv_dim if w.conv_dim > 0 else 2 * HK * S + H * S
    K = w.conv_kernel
    rng = np.random.default_rng(w.seed if seed is None else seed)
    d = {}
    d["q_raw"] = normal(rng, (N, T, HK, S))
    d["k_raw"] = normal(rng, (N, T, HK, S))
    d["v"] = normal(rng, (N, T, H, S))
    d["a"] = normal(rng, (N, T, H))
    d["b"] = normal(rng, (N, T, H))
    d["A_log"] = normal(rng, (H,))
    d["dt_bias"] = np.zeros((H,), dtype=np.float32)
    if w.state_sigma > 0:
        d["state"] = normal(rng, (N, H, S, S), w.state_sigma)
    else:
        d["state"] = np.zeros((N, H, S, S), dtype=np.float32)
    if conv:
        d["conv_w"] = normal(rng, (C, K), 0.5)
        if w.conv_state_sigma > 0:
            d["conv_state"] = normal(rng, (N, C, K - 1), w.conv_state_sigma)
        else:
            d["conv_state"] = np.zeros((N, C, K - 1), dtype=np.float32)
        d["x"] = normal(rng, (N, T, C))
    d["norm_w"] = normal(rng, (S,), 0.1, 1.0)
    d["z"] = normal(rng, (N, T, H, S))
    return d


def draw_block_layer(layer: int, w: Workload | int = 4, n_seqs: int | None = None) -> dict:
    """Raw draws for one layer of the bf16 decode block (64 sequences x 48 layers).

    Returns qkv [N][C] and z [N][H][S] as bf16 bit patterns (uint16) plus
    float32 a, b [N][H], conv_w [C][K], A_log, dt_bias [H], norm_w [S],
    conv_state [N][C][K-1] and state [N][H][S][S].
    """
    if isinstance(w, int):
        w = WORKLOADS[w]
    N = w.n_seqs if n_seqs is None else n_seqs
    H, HK, S, K = w.n_v_heads, w.n_k_heads, w.state_size, w.conv_kernel
    C = 2 * HK * S + H * S
    rng = np.random.default_rng(w.seed + layer)
    d = {}
    d["a"] = normal(rng, (N, H))
    d["b"] = normal(rng, (N, H))
    d["A_log"] = normal(rng, (H,))
    d["dt_bias"] = np.zeros((H,), dtype=np.float32)
    d["state"] = normal(rng, (N, H, S, S), w.state_sigma)
    d["conv_w"] = normal(rng, (C, K), 0.5)
    d["conv_state"] = normal(rng, (N, C, K - 1), w.conv_state_sigma)
    d["qkv"] = to_bf16_bits(normal(rng, (N, C)))   # the conv input "x"
    d["norm_w"] = normal(rng, (S,), 0.1, 1.0)
    d["z"] = to_bf16_bits(normal(rng, (N, H, S)))
    return d


def draw_prefill(seed: int = 6, n_seqs: int = 1, n_tokens: int = 4096, n_k_heads: int = 16,
                 n_v_heads: int = 32, state_size: int = 128, conv_kernel: int = 4,
                 state_sigma: float = 0.0, conv_state_sigma: float = 0.0) -> dict:
    """Raw draws for one prefill layer: qkv [N][T][C] and z [N][T][H][S] as bf16
    bit patterns; a, b [N][T][H]; A_log, dt_bias (zeros) [H]; state
    [N][H][S][S]; conv_w [C][K]; conv_state [N][C][K-1]; norm_w [S]. Drawn in
    the module's order (a, b, A_log, state, conv_w, conv_state, x, norm_w, z)."""
    N, T, HK, H, S, K = n_seqs, n_tokens, n_k_heads, n_v_heads, state_size, conv_kernel
    C = 2 * HK * S + H * S
    rng = np.random.default_rng(seed)
    d = {}
    d["a"] = normal(rng, (N, T, H))
    d["b"] = normal(rng, (N, T, H))
    d["A_log"] = normal(rng, (H,))
    d["dt_bias"] = np.zeros((H,), dtype=np.float32)
    d["state"] = (normal(rng, (N, H, S, S), state_sigma) if state_sigma > 0
                  else np.zeros((N, H, S, S), dtype=np.float32))
    d["conv_w"] = normal(rng, (C, K), 0.5)
    d["conv_state"] = (normal(rng, (N, C, K - 1), conv_state_sigma) if conv_state_sigma > 0
                       else np.zeros((N, C, K - 1), dtype=np.float32))
    d["qkv"] = to_bf16_bits(normal(rng, (N, T, C)))
    d["norm_w"] = normal(rng, (S,), 0.1, 1.0)
    d["z"] = to_bf16_bits(normal(rng, (N, T, H, S)))
    return d
