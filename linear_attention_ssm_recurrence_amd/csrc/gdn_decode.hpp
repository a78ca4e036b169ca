// The batched decode kernel of the gated delta-rule recurrence on gfx950 (one
// token per sequence). Included by gdn_recurrence.hip, which holds the entry
// points; kept in a header of its own so that the decode's measured traffic
// (recorded with a hash of this file and gdn_device.hpp) stays tied to the
// decode's own source.
#pragma once

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// Decode: each wave owns RW consecutive rows of one (sequence, head). It
// issues every state load of its rows first (RW/G * E/4 float4 loads per
// lane, all independent, non-temporal: the state is touched once per launch),
// then runs the step row-group by row-group and streams the rows back with
// non-temporal stores. k and q of the head are loaded once per wave and reused
// for all its rows; g and beta are wave-uniform. Small waves (8 rows, 4 KiB of
// state) in 8-wave blocks keep the most requests in flight across the chip:
// measured on MI355X at S = 128 this streams faster than 16- or 32-row waves
// and than a plain non-temporal copy kernel.
// ---------------------------------------------------------------------------
constexpr int kDecodeWaves = 8;

// With T4 the read-out is regrouped as y = scale * (r_dec . q + delta * qk)
// (delta_rule_step_t4); qk = k . q is reduced once per wave, in qk_dot's
// order, which the scan's T4 form shares. The state is the
// same either way. V-head h of sequence n reads K-head h mod n_k_heads of q
// and k (the tiled grouped-query repeat), so q and k are [N][HK][S].
template <int S, int RW, bool T4>
__global__ __launch_bounds__(64 * kDecodeWaves) void recurrence_decode_kernel(
    float* __restrict__ state, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ y, int64_t n_pairs, int n_k_heads, int n_v_heads, float scale) {
  using Lay = RecurLayout<S>;
  constexpr int E = Lay::E, L = Lay::L, G = Lay::G;
  constexpr int IT = RW / G;         // row groups per wave
  constexpr int WPH = S / RW;        // waves per (sequence, head)
  static_assert(RW % G == 0 && S % RW == 0, "rows per wave must tile the head");

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t pair = wave / WPH;   // n * H + h
  if (pair >= n_pairs) return;  // uniform across the wave; the kernel has no barrier
  const int p = lane % L;
  const int row0 = (int)(wave % WPH) * RW + lane / L;
  const int64_t kq = (pair / n_v_heads) * n_k_heads + (pair % n_v_heads) % n_k_heads;

  float kk[E], qq[E];
  load_row_part<E, L>(k + kq * S, p, kk);
  load_row_part<E, L>(q + kq * S, p, qq);
  const float d = expf(g[pair]);
  const float b = beta[pair];
  float qk = 0.0f;
  if constexpr (T4) {   // k . q in qk_dot's order: lane i of each group of S/4 takes entries 4i..4i+3
    const int i4 = 4 * (lane % (S / 4));
    qk = qk_dot<S>(load4(k + kq * S + i4), load4(q + kq * S + i4));
  }

  float* sp = state + pair * (int64_t)S * S;
  float4 raw[IT][E / 4];
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int m = 0; m < E / 4; ++m)
      raw[it][m] = load4_stream(sp + (int64_t)(row0 + it * G) * S + 4 * (p + L * m));
  float vv[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) vv[it] = v[pair * S + row0 + it * G];

#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float r[E];
    unpack<E>(raw[it], r);
    float yj;
    if constexpr (T4)
      yj = delta_rule_step_t4<E, L>(r, kk, qq, vv[it], d, b, qk, scale);
    else
      yj = delta_rule_step<E, L>(r, kk, qq, vv[it], d, b, scale);
    float* rp = sp + (int64_t)(row0 + it * G) * S;
#pragma unroll
    for (int m = 0; m < E / 4; ++m)
      store4_stream(rp + 4 * (p + L * m), make_float4(r[4 * m], r[4 * m + 1], r[4 * m + 2], r[4 * m + 3]));
    if (p == 0) y[pair * S + row0 + it * G] = yj;
  }
}

template <int S>
struct DecodeCfg;
template <> struct DecodeCfg<32> { static constexpr int RW = 16; };   // G = 16 rows per slot
template <> struct DecodeCfg<64> { static constexpr int RW = 8; };
template <> struct DecodeCfg<128> { static constexpr int RW = 8; };
template <> struct DecodeCfg<256> { static constexpr int RW = 8; };

template <int S, bool T4>
static int launch_decode(float* state, const float* q, const float* k, const float* v,
                         const float* g, const float* beta, float* y, int n_seqs, int n_k_heads,
                         int n_v_heads, float scale, hipStream_t stream) {
  constexpr int RW = DecodeCfg<S>::RW;
  const int64_t n_pairs = (int64_t)n_seqs * n_v_heads;
  const int64_t waves = n_pairs * (S / RW);
  const unsigned blocks = grid_for(waves, kDecodeWaves);
  return launch(recurrence_decode_kernel<S, RW, T4>, dim3(blocks), dim3(64 * kDecodeWaves),
                0, stream, state, q, k, v, g, beta, y, n_pairs, n_k_heads, n_v_heads, scale);
}

}  // namespace gdn
