// One decode step of the gated delta rule from the raw per-token inputs, in
// one kernel: the q/k L2 norm with the tiled grouped-query repeat, the decay
// gate, beta = sigmoid(b), and the recurrence step (the "glue" kernels of
// ssm_gated_delta.cu's decode path folded into its recurrence kernel, with the
// repeat by index of mlx-native gated_delta_net_decode.metal).
//
// The kernel is the batched decode kernel (gdn_decode.hpp) with its inputs
// formed in registers: each 16-lane row group of a wave (S = 128) already
// holds the whole q and k of its K-head, E = 8 floats per lane in two float4
// slots, so the sums of squares need no LDS and no barrier. They are formed in
// the order of row_sumsq, the reduction of the stand-alone L2-norm kernel:
// there, lane m of a wave holds float4 slot m of the head (m < S/4), squares
// it into a four-term FMA chain, and the wave sums the chains with
// group_sum<64>. Here a lane holds slots p and p + L (L = S/8 lanes per row);
// group_sum<L> over each slot separately gives the two halves of that
// butterfly (its first log2(L) steps never mix them), and their sum is its
// next step; the remaining steps of group_sum<64> only add +0. The decay
// gate, exp, and sigmoid are the shared device functions. So this kernel
// equals gdn_l2norm_gqa + gdn_decay_gate + gdn_sigmoid + gdn_recurrence bit
// for bit, in one launch instead of four.
#include "gdn_decode.hpp"

namespace gdn {

#pragma clang fp contract(off)

// x / max(||x||, eps) of a head held in the decode layout (slots p and p + L
// of every lane of an L-lane row group), summed in row_sumsq's order.
template <int E, int L>
__device__ __forceinline__ void l2_normalise_row(float (&x)[E], float eps) {
  static_assert(E == 8, "two float4 slots per lane");
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s0 = __builtin_fmaf(x[e], x[e], s0);
#pragma unroll
  for (int e = 4; e < 8; ++e) s1 = __builtin_fmaf(x[e], x[e], s1);
  const float ss = group_sum<L>(s0) + group_sum<L>(s1);
  const float inv = inv_l2norm(ss, eps);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = x[e] * inv;
}

template <int S, int RW>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_step_kernel(
    float* __restrict__ state, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ a, const float* __restrict__ b,
    const float* __restrict__ ssm_a, const float* __restrict__ dt_bias, float* __restrict__ y,
    int64_t n_pairs, int n_k_heads, int n_v_heads, float scale, float l2_eps) {
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
  const int h = (int)(pair % n_v_heads);
  const int64_t kq = (pair / n_v_heads) * n_k_heads + h % n_k_heads;

  // the raw q, k of the K-head and the gate inputs first, then the state rows:
  // the norms and the gate are formed while the state is in flight
  float kk[E], qq[E];
  load_row_part<E, L>(k + kq * S, p, kk);
  load_row_part<E, L>(q + kq * S, p, qq);
  const float av = a[pair], bv = b[pair], dtb = dt_bias[h], sa = ssm_a[h];
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

  l2_normalise_row<E, L>(kk, l2_eps);
  l2_normalise_row<E, L>(qq, l2_eps);
  const float d = expf(decay_gate(av, dtb, sa));
  const float bt = sigmoid(bv);

#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float r[E];
    unpack<E>(raw[it], r);
    const float yj = delta_rule_step<E, L>(r, kk, qq, vv[it], d, bt, scale);
    float* rp = sp + (int64_t)(row0 + it * G) * S;
#pragma unroll
    for (int m = 0; m < E / 4; ++m)
      store4_stream(rp + 4 * (p + L * m), make_float4(r[4 * m], r[4 * m + 1], r[4 * m + 2], r[4 * m + 3]));
    if (p == 0) y[pair * S + row0 + it * G] = yj;
  }
}

template <int S>
static int launch_decode_step(float* state, const float* q, const float* k, const float* v,
                              const float* a, const float* b, const float* ssm_a,
                              const float* dt_bias, float* y, int n_seqs, int n_k_heads,
                              int n_v_heads, float scale, float l2_eps, hipStream_t stream) {
  constexpr int RW = DecodeCfg<S>::RW;
  const int64_t n_pairs = (int64_t)n_seqs * n_v_heads;
  const int64_t waves = n_pairs * (S / RW);
  return launch(decode_step_kernel<S, RW>, dim3(grid_for(waves, kDecodeWaves)),
                dim3(64 * kDecodeWaves), 0, stream, state, q, k, v, a, b, ssm_a, dt_bias, y,
                n_pairs, n_k_heads, n_v_heads, scale, l2_eps);
}

}  // namespace gdn

using namespace gdn;

extern "C" int gdn_decode_step(float* state, const float* q, const float* k, const float* v,
                               const float* a, const float* b, const float* ssm_a,
                               const float* dt_bias, float* y, int n_seqs, int n_k_heads,
                               int n_v_heads, int state_size, float scale, float l2_eps,
                               void* stream) {
  if (n_seqs < 0 || n_k_heads <= 0 || n_v_heads <= 0 || state_size <= 0) return GDN_ESIZE;
  if (n_v_heads % n_k_heads != 0) return GDN_ESIZE;
  if (!is_state_size(state_size)) return GDN_EUNSUPPORTED;
  if (n_seqs == 0) return GDN_OK;
  if (!state || !q || !k || !v || !a || !b || !ssm_a || !dt_bias || !y) return GDN_ENULL;
  int64_t pairs, st;
  if (!mul_ok(n_seqs, n_v_heads, &pairs) || !mul_ok(pairs, (int64_t)state_size * state_size, &st))
    return GDN_ESIZE;
  if (pairs * (state_size / 8) / kDecodeWaves >= (int64_t(1) << 31)) return GDN_ESIZE;
  if (!aligned16(state) || !aligned16(q) || !aligned16(k)) return GDN_EALIGN;
  hipStream_t s = as_stream(stream);
  switch (state_size) {
    case 32: return launch_decode_step<32>(state, q, k, v, a, b, ssm_a, dt_bias, y, n_seqs, n_k_heads, n_v_heads, scale, l2_eps, s);
    case 64: return launch_decode_step<64>(state, q, k, v, a, b, ssm_a, dt_bias, y, n_seqs, n_k_heads, n_v_heads, scale, l2_eps, s);
    case 128: return launch_decode_step<128>(state, q, k, v, a, b, ssm_a, dt_bias, y, n_seqs, n_k_heads, n_v_heads, scale, l2_eps, s);
    case 256: return launch_decode_step<256>(state, q, k, v, a, b, ssm_a, dt_bias, y, n_seqs, n_k_heads, n_v_heads, scale, l2_eps, s);
  }
  return GDN_EUNSUPPORTED;
}
