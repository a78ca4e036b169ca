// One decode layer of the Gated DeltaNet block fused into a single gfx950
// kernel: bf16 activations, fp32 state.
//
// Per sequence the layer runs conv1d + SiLU over all channels, splits the
// result as [q | k | v], L2-normalises q and k per K-head, repeats them to the
// V-heads by index (V-head vh reads K-head vh mod HK), computes beta = sigmoid(b)
// and the decay gate, takes one delta-rule step per state row, and applies the
// gated RMSNorm to the read-out (the decode order of ssm_gated_delta.cu's
// file header and "glue" kernels, with the tiled repeat of mlx-native
// gated_delta_net_decode.metal).
//
// Work split. One workgroup of 8 waves owns (sequence n, K-head kh) and with
// it every V-head vh = kh + r*HK (r < GQ = H/HK). The conv channels those
// heads read (q and k of kh, v of each vh) are read by no other workgroup, so
// each channel's history is rolled exactly once. The workgroup:
//   0. issues the small loads of phases 1-2 and 4 (conv, gate and norm inputs), then
//      the loads of all its state rows (GQ*S rows, 64 KiB per V-head), so
//      that the state's HBM transfer overlaps phases 1-2 (the hardware
//      counts outstanding loads in issue order: loads issued after the state
//      would have to wait for all of it);
//   1. convolves its (2 + GQ)*S channels into LDS and rolls their history;
//   2. L2-normalises q and k in LDS (waves 0 and 1); wave 2 computes beta and
//      exp(g) of the GQ V-heads;
//   3. runs the delta-rule step on its rows (each wave holds GQ*S/8 rows)
//      and writes y to LDS;
//   4. gated-RMSNorms each V-head's y with z (waves 0..GQ-1) and stores it.
// Every step uses the same device function as the stand-alone kernel of that
// step, so the layer equals the stand-alone kernels chained, bit for bit.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kBlockS = 128;
constexpr int kBlockWaves = 8;

template <int GQ, int K>
__global__ __launch_bounds__(64 * kBlockWaves) void decode_block_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ z, const float* __restrict__ a,
    const float* __restrict__ b, const float* __restrict__ conv_w,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const float* __restrict__ norm_w, float* __restrict__ conv_state, float* __restrict__ state,
    float* __restrict__ out, int n_k_heads, float scale, float l2_eps, float eps) {
  constexpr int S = kBlockS;
  using Lay = RecurLayout<S>;
  constexpr int E = Lay::E, L = Lay::L, G = Lay::G;
  constexpr int RW = GQ * S / kBlockWaves;  // state rows per wave
  constexpr int IT = RW / G;                // row groups per wave
  constexpr int NCH = (2 + GQ) * S;         // conv channels of the workgroup
  static_assert(RW % G == 0 && S % RW == 0, "a wave's rows must lie in one V-head");

  __shared__ float co[NCH];      // conv output: q | k | v[0..GQ)
  __shared__ float ys[GQ * S];   // read-out of each V-head
  __shared__ float gate_d[GQ];   // exp(g)
  __shared__ float gate_b[GQ];   // beta

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n_v_heads = GQ * n_k_heads;
  const int key_dim = n_k_heads * S;
  const int64_t C = 2 * (int64_t)key_dim + (int64_t)n_v_heads * S;
  const int kh = blockIdx.x % n_k_heads;
  const int64_t n = blockIdx.x / n_k_heads;

  // 0a. inputs of the conv (channels ch = tid + ci * threads) and of the gate
  constexpr int TPB = 64 * kBlockWaves;
  constexpr int CPT = (NCH + TPB - 1) / TPB;      // conv channels per thread
  float wc[CPT][K], hist[CPT][K - 1], xv[CPT];
  float* csp[CPT];
#pragma unroll
  for (int ci = 0; ci < CPT; ++ci) {
    const int ch = tid + ci * TPB;
    if (ch < NCH) {
      const int seg = ch / S, i = ch % S;
      int64_t c;
      if (seg == 0) c = (int64_t)kh * S + i;
      else if (seg == 1) c = key_dim + (int64_t)kh * S + i;
      else c = 2 * (int64_t)key_dim + (int64_t)(kh + (seg - 2) * n_k_heads) * S + i;
#pragma unroll
      for (int u = 0; u < K; ++u) wc[ci][u] = conv_w[c * K + u];
      csp[ci] = conv_state + (n * C + c) * (K - 1);
#pragma unroll
      for (int u = 0; u < K - 1; ++u) hist[ci][u] = csp[ci][u];
      xv[ci] = bf16_to_float(qkv[n * C + c]);
    }
  }
  const bool gate_lane = (wv == 2 && lane < GQ);
  float ga = 0.0f, gdt = 0.0f, gal = 0.0f, gb = 0.0f;
  if (gate_lane) {
    const int h = kh + lane * n_k_heads;
    ga = a[n * n_v_heads + h];
    gdt = dt_bias[h];
    gal = A_log[h];
    gb = b[n * n_v_heads + h];
  }

  // 0a'. z and norm_w of the gated norm (waves 0..GQ-1, one float4 group of
  // the head's row per lane), so that phase 4 waits on no global load: the
  // next workgroup on this CU needs the slots of waves 0..GQ-1 as well
  static_assert(S / 4 <= 64, "one float4 group of a norm row per lane");
  const bool norm_lane = (wv < GQ && lane < S / 4);
  uint2 zb_pre = make_uint2(0u, 0u);
  float4 nw_pre = make_float4(0.f, 0.f, 0.f, 0.f);
  if (norm_lane) {
    const int h = kh + wv * n_k_heads;
    zb_pre = *reinterpret_cast<const uint2*>(z + (n * n_v_heads + h) * S + 4 * lane);
    nw_pre = load4(norm_w + 4 * lane);
  }

  // 0b. state rows of this wave: combined row R = wv*RW + ... over the GQ heads
  const int r_head = (wv * RW) / S;                 // which of the GQ V-heads
  const int vh = kh + r_head * n_k_heads;
  const int p = lane % L;
  const int row0 = (wv * RW) % S + lane / L;        // row j within the V-head
  float* sp = state + (n * n_v_heads + vh) * (int64_t)S * S;
  float4 raw[IT][E / 4];
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int m = 0; m < E / 4; ++m)
      raw[it][m] = load4_stream(sp + (int64_t)(row0 + it * G) * S + 4 * (p + L * m));

  // 1. conv of the workgroup's channels
#pragma unroll
  for (int ci = 0; ci < CPT; ++ci) {
    const int ch = tid + ci * TPB;
    if (ch < NCH) {
      co[ch] = conv_point<K>(xv[ci], hist[ci], wc[ci]);
#pragma unroll
      for (int u = 0; u + 1 < K - 1; ++u) csp[ci][u] = hist[ci][u + 1];
      csp[ci][K - 2] = xv[ci];
    }
  }
  __syncthreads();

  // 2. L2 norm of q (wave 0) and k (wave 1); gate and beta (wave 2)
  if (wv < 2) {
    float* x = co + wv * S;
    const float ss = row_sumsq(x, S / 4, lane);
    const float norm = sqrtf(ss);
    const float inv = 1.0f / (norm > l2_eps ? norm : l2_eps);
    for (int m = lane; m < S / 4; m += 64) {
      float4 v = load4(x + 4 * m);
      v.x = v.x * inv;
      v.y = v.y * inv;
      v.z = v.z * inv;
      v.w = v.w * inv;
      store4(x + 4 * m, v);
    }
  } else if (gate_lane) {
    const float gv = decay_gate(ga, gdt, gal);
    gate_d[lane] = expf(gv);
    gate_b[lane] = sigmoid(gb);
  }
  __syncthreads();

  // 3. delta-rule step on this wave's rows
  {
    float kk[E], qq[E];
    load_row_part<E, L>(co + S, p, kk);
    load_row_part<E, L>(co, p, qq);
    const float d = gate_d[r_head];
    const float bt = gate_b[r_head];
    const float* vv = co + (2 + r_head) * S;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float r[E];
      unpack<E>(raw[it], r);
      const int j = row0 + it * G;
      const float yj = delta_rule_step<E, L>(r, kk, qq, vv[j], d, bt, scale);
      float* rp = sp + (int64_t)j * S;
#pragma unroll
      for (int m = 0; m < E / 4; ++m)
        store4_stream(rp + 4 * (p + L * m),
                      make_float4(r[4 * m], r[4 * m + 1], r[4 * m + 2], r[4 * m + 3]));
      if (p == 0) ys[r_head * S + j] = yj;
    }
  }
  __syncthreads();

  // 4. gated RMSNorm of each V-head's read-out
  if (wv < GQ) {
    const int h = kh + wv * n_k_heads;
    const float* yr = ys + wv * S;
    const float ss = row_sumsq(yr, S / 4, lane);
    const float inv = 1.0f / sqrtf(ss / (float)S + eps);
    float* orow = out + (n * n_v_heads + h) * S;
    if (norm_lane) {
      const int m = lane;
      const float4 yv = load4(yr + 4 * m);
      const float4 wv4 = nw_pre;
      const uint2 zb = zb_pre;
      const float z0 = bf16_to_float((uint16_t)(zb.x & 0xFFFFu));
      const float z1 = bf16_to_float((uint16_t)(zb.x >> 16));
      const float z2 = bf16_to_float((uint16_t)(zb.y & 0xFFFFu));
      const float z3 = bf16_to_float((uint16_t)(zb.y >> 16));
      float4 o;
      o.x = yv.x * inv * wv4.x * silu(z0);
      o.y = yv.y * inv * wv4.y * silu(z1);
      o.z = yv.z * inv * wv4.z * silu(z2);
      o.w = yv.w * inv * wv4.w * silu(z3);
      store4(orow + 4 * m, o);
    }
  }
}

template <int GQ, int K>
static int launch_block(const uint16_t* qkv, const uint16_t* z, const float* a, const float* b,
                        const float* conv_w, const float* A_log, const float* dt_bias,
                        const float* norm_w, float* conv_state, float* state, float* out,
                        int n_seqs, int n_k_heads, float scale, float l2_eps, float eps,
                        hipStream_t s) {
  const int64_t blocks = (int64_t)n_seqs * n_k_heads;
  hipLaunchKernelGGL((decode_block_kernel<GQ, K>), dim3((unsigned)blocks), dim3(64 * kBlockWaves),
                     0, s, qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state, state, out,
                     n_k_heads, scale, l2_eps, eps);
  return launch_status();
}

template <int GQ>
static int launch_block_k(int K, const uint16_t* qkv, const uint16_t* z, const float* a,
                          const float* b, const float* conv_w, const float* A_log,
                          const float* dt_bias, const float* norm_w, float* conv_state,
                          float* state, float* out, int n_seqs, int n_k_heads, float scale,
                          float l2_eps, float eps, hipStream_t s) {
  switch (K) {
    case 2: return launch_block<GQ, 2>(qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
    case 3: return launch_block<GQ, 3>(qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
    case 4: return launch_block<GQ, 4>(qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
  }
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn

using namespace gdn;

extern "C" int gdn_decode_block_bf16(const uint16_t* qkv, const uint16_t* z, const float* a,
                                     const float* b, const float* conv_w, const float* A_log,
                                     const float* dt_bias, const float* norm_w,
                                     float* conv_state, float* state, float* out, int n_seqs,
                                     int n_k_heads, int n_v_heads, int state_size,
                                     int conv_kernel, float scale, float l2_eps, float eps,
                                     void* stream) {
  if (n_seqs < 0 || n_k_heads <= 0 || n_v_heads <= 0 || state_size <= 0 || conv_kernel <= 0)
    return GDN_ESIZE;
  if (n_v_heads % n_k_heads != 0) return GDN_ESIZE;
  const int gq = n_v_heads / n_k_heads;
  if (state_size != kBlockS || !(gq == 1 || gq == 2 || gq == 4)) return GDN_EUNSUPPORTED;
  if (conv_kernel < 2 || conv_kernel > 4) return GDN_EUNSUPPORTED;
  if (n_seqs == 0) return GDN_OK;
  if (!qkv || !z || !a || !b || !conv_w || !A_log || !dt_bias || !norm_w || !conv_state ||
      !state || !out)
    return GDN_ENULL;
  int64_t pairs, st;
  if (!mul_ok(n_seqs, n_v_heads, &pairs) || !mul_ok(pairs, (int64_t)state_size * state_size, &st))
    return GDN_ESIZE;
  if ((int64_t)n_seqs * n_k_heads >= (int64_t(1) << 31)) return GDN_ESIZE;
  if (!aligned16(state) || !aligned16(norm_w) || !aligned16(out)) return GDN_EALIGN;
  if ((reinterpret_cast<uintptr_t>(z) & 7u) != 0) return GDN_EALIGN;
  hipStream_t s = as_stream(stream);
  switch (gq) {
    case 1: return launch_block_k<1>(conv_kernel, qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
    case 2: return launch_block_k<2>(conv_kernel, qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
    case 4: return launch_block_k<4>(conv_kernel, qkv, z, a, b, conv_w, A_log, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
  }
  return GDN_EUNSUPPORTED;
}
