// Device-side building blocks shared by the gfx950 kernels of the Gated
// DeltaNet block: wave64 segmented reductions, the per-row delta-rule step,
// and the scalar functions of the block (SiLU, guarded softplus, sigmoid).
//
// Floating-point contraction is off in this header's functions: every fused
// multiply-add is written explicitly, so the instruction sequence (and hence
// the bits) of a step does not depend on the kernel it is inlined into. That
// is what makes the scan kernel and chained decode launches agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// ---------------------------------------------------------------------------
// Cross-lane moves
// ---------------------------------------------------------------------------

// DPP move within a row of 16 lanes; every lane reads a lane of its own row,
// so no lane is ever left without a source.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

// Exchange with lane ^ 16 inside each 32-lane half (ds_swizzle, bit-mask mode:
// and_mask 0x1F, or_mask 0, xor_mask 0x10).
__device__ __forceinline__ float swizzle_xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// Exchange with lane ^ 32 (crosses the two halves of the wave).
__device__ __forceinline__ float bpermute_xor32(float v) {
  const int lane = __lane_id();
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, v)));
}

// Sum over each aligned group of L consecutive lanes (L a power of two, 1..64),
// returned in every lane of the group. Each step adds a lane's value to its
// partner's, and the two partners form the same sum (fp addition commutes),
// so all lanes of a group hold identical bits.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16 || L == 32 || L == 64,
                "group size must be a power of two up to 64");
  if constexpr (L >= 2) v = v + dpp_mov<kDppQuadXor1>(v);
  if constexpr (L >= 4) v = v + dpp_mov<kDppQuadXor2>(v);
  if constexpr (L >= 8) v = v + dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (L >= 16) v = v + dpp_mov<kDppRowMirror>(v);
  if constexpr (L >= 32) v = v + swizzle_xor16(v);
  if constexpr (L >= 64) v = v + bpermute_xor32(v);
  return v;
}

// ---------------------------------------------------------------------------
// Scalar functions
// ---------------------------------------------------------------------------

#pragma clang fp contract(off)

// SiLU in the divisor form x / (1 + e^-x) (the form both Foundry pages use),
// in five instructions: e^-x as the hardware base-2 exponential of
// -x*log2(e) (v_exp_f32), then x times the hardware reciprocal of 1 + e^-x
// (v_rcp_f32). Rounding the product -x*log2(e) perturbs e^-x by at most
// |x|*7e-8 relative, and each hardware instruction adds about one ulp, so the
// result is within about 1e-7 of the exact SiLU in absolute terms and
// (|x|*7e-8 + 4e-7) relative: far inside the tolerance, and unlike the decay's
// exp this error does not compound (a SiLU output feeds no recurrence of its
// own). For x below about -88, e^-x is +inf, its reciprocal +0, and the result
// -0, as with the IEEE quotient. Every kernel uses this one function, so the
// kernels agree with each other bit for bit.
__device__ __forceinline__ float silu(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// 1 / max(||x||, eps) from the sum of squares ss = ||x||^2 of an L2 norm:
// the hardware reciprocal square root (v_rsq_f32, about one ulp) of
// max(ss, eps^2), which has the same value up to rounding (max(sqrt(ss), eps)
// = sqrt(max(ss, eps^2))). A NaN ss takes eps^2, as the comparison form takes
// eps. Every L2 norm of the library uses this one function.
__device__ __forceinline__ float inv_l2norm(float ss, float eps) {
  return __builtin_amdgcn_rsqf(fmaxf(ss, eps * eps));
}

// Logistic sigmoid 1 / (1 + e^-x).
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// softplus(u) = log(1 + e^u), passed through unchanged above 20 so that e^u
// cannot overflow (an infinite softplus would zero the decay and wipe the
// head's state).
__device__ __forceinline__ float softplus_guarded(float u) {
  return u > 20.0f ? u : log1pf(expf(u));
}

// g = ssm_a * softplus(a + dt_bias), with ssm_a = -exp(A_log) <= 0 prepared
// once per head by the caller (gdn_ssm_a), as both Foundry pages pre-bake it.
__device__ __forceinline__ float decay_gate(float a, float dt_bias, float ssm_a) {
  return ssm_a * softplus_guarded(a + dt_bias);
}

// ssm_a = -exp(A_log): the per-head factor of the decay gate.
__device__ __forceinline__ float ssm_a_of(float A_log) { return -expf(A_log); }

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_float(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// ---------------------------------------------------------------------------
// The delta-rule step on one state row
// ---------------------------------------------------------------------------
//
// A row of S floats is spread over L = S / E consecutive lanes, E floats per
// lane in E/4 float4 slots: lane position p (0..L-1) holds, in slot m, the
// four row entries 4*(p + L*m) .. 4*(p + L*m) + 3. One float4 access of a
// slot therefore covers 16*L contiguous bytes of the row.

// Row layout of the recurrence kernels for each state size S: E floats per
// lane, L lanes per row, G rows per wave per float4 slot. The decode, scan
// and fused-block kernels all use it, which is what keeps them bit-identical.
template <int S>
struct RecurLayout {
  static constexpr int E = 8;
  static constexpr int L = S / E;
  static constexpr int G = 64 / L;
};

// In-lane part of a dot product, in a fixed order: two accumulation chains
// (even and odd entries), then their sum.
template <int E>
__device__ __forceinline__ float lane_dot(const float (&a)[E], const float (&b)[E]) {
  static_assert(E % 2 == 0, "E must be even");
  float p0 = a[0] * b[0];
  float p1 = a[1] * b[1];
#pragma unroll
  for (int e = 2; e < E; e += 2) {
    p0 = __builtin_fmaf(a[e], b[e], p0);
    p1 = __builtin_fmaf(a[e + 1], b[e + 1], p1);
  }
  return p0 + p1;
}

// One token of the gated delta rule on one row (the lane's E entries of it):
//   r = d * r; pred = r . k; delta = (v - pred) * beta; r = r + k * delta;
//   returns scale * (r . q), the read-out after the update.
// v, d, beta and scale are the same in all L lanes of the row; the result is
// identical in all of them.
template <int E, int L>
__device__ __forceinline__ float delta_rule_step(float (&r)[E], const float (&k)[E],
                                                 const float (&q)[E], float v, float d, float beta,
                                                 float scale) {
#pragma unroll
  for (int e = 0; e < E; ++e) r[e] = r[e] * d;
  const float pred = group_sum<L>(lane_dot<E>(r, k));
  const float delta = (v - pred) * beta;
#pragma unroll
  for (int e = 0; e < E; ++e) r[e] = __builtin_fmaf(k[e], delta, r[e]);
  const float o = group_sum<L>(lane_dot<E>(r, q));
  return scale * o;
}

// k . q of one head and token for the "T4" read-out, in one fixed order that
// every kernel using it shares: each lane of an aligned group of S/4 lanes
// holds the four consecutive entries 4i .. 4i+3 (i its index in the group),
// forms a four-term chain, and the group sums the chains. Every lane of the
// group returns the same bits.
template <int S>
__device__ __forceinline__ float qk_dot(float4 k, float4 q) {
  static_assert(S % 4 == 0 && S / 4 <= 64, "a head must fit one group of lanes");
  float p = k.x * q.x;
  p = __builtin_fmaf(k.y, q.y, p);
  p = __builtin_fmaf(k.z, q.z, p);
  p = __builtin_fmaf(k.w, q.w, p);
  return group_sum<S / 4>(p);
}

// The same token with the read-out regrouped as in the "T4" kernel of
// ssm_gated_delta.cu (fc_ssm_recurrence_slots_2pass): after the decay,
//   y = scale * (r_dec . q + delta * (k . q)),
// so pred = r_dec . k and r_dec . q are reduced together from the decayed row
// and no dot product waits on the update. qk = k . q is the same for every row
// of the head and is passed in. The state trajectory is identical to
// delta_rule_step's bit for bit; only y is reassociated.
template <int E, int L>
__device__ __forceinline__ float delta_rule_step_t4(float (&r)[E], const float (&k)[E],
                                                    const float (&q)[E], float v, float d, float beta,
                                                    float qk, float scale) {
#pragma unroll
  for (int e = 0; e < E; ++e) r[e] = r[e] * d;
  const float pred = group_sum<L>(lane_dot<E>(r, k));
  const float oq = group_sum<L>(lane_dot<E>(r, q));
  const float delta = (v - pred) * beta;
#pragma unroll
  for (int e = 0; e < E; ++e) r[e] = __builtin_fmaf(k[e], delta, r[e]);
  return scale * __builtin_fmaf(delta, qk, oq);
}

// One output of the causal conv1d + SiLU: the newest tap first,
// x * w[K-1], then history[u] * w[u] for ascending u (oldest first), then SiLU.
template <int K>
__device__ __forceinline__ float conv_point(float x, const float (&hist)[K - 1], const float (&w)[K]) {
  float acc = x * w[K - 1];
#pragma unroll
  for (int u = 0; u < K - 1; ++u) acc = __builtin_fmaf(hist[u], w[u], acc);
  return silu(acc);
}

#pragma clang fp contract(off)
// Sum of squares of a row of D floats (d4 = D/4 float4 slots) spread over a
// wave: lane reads slots lane, lane + 64, ...; the wave then reduces.
__device__ __forceinline__ float row_sumsq(const float* row, int d4, int lane) {
  float s = 0.0f;
  for (int m = lane; m < d4; m += 64) {
    const float4 v = *reinterpret_cast<const float4*>(row + 4 * m);
    s = __builtin_fmaf(v.x, v.x, s);
    s = __builtin_fmaf(v.y, v.y, s);
    s = __builtin_fmaf(v.z, v.z, s);
    s = __builtin_fmaf(v.w, v.w, s);
  }
  return group_sum<64>(s);
}

#pragma clang fp contract(fast)

// ---------------------------------------------------------------------------
// Vector memory helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) float4 access, for data touched once per launch.
__device__ __forceinline__ float4 load4_stream(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store4_stream(float* p, float4 v) {
  const f32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}

template <int E>
__device__ __forceinline__ void unpack(const float4 (&v)[E / 4], float (&r)[E]) {
#pragma unroll
  for (int m = 0; m < E / 4; ++m) {
    r[4 * m + 0] = v[m].x;
    r[4 * m + 1] = v[m].y;
    r[4 * m + 2] = v[m].z;
    r[4 * m + 3] = v[m].w;
  }
}

template <int E, int L>
__device__ __forceinline__ void load_row_part(const float* row, int p, float (&r)[E]) {
#pragma unroll
  for (int m = 0; m < E / 4; ++m) {
    const float4 v = load4(row + 4 * (p + L * m));
    r[4 * m + 0] = v.x;
    r[4 * m + 1] = v.y;
    r[4 * m + 2] = v.z;
    r[4 * m + 3] = v.w;
  }
}

}  // namespace gdn
