// Companion steps of the Gated DeltaNet block on gfx950: the decay gate, the
// sigmoid of beta, the q/k L2 normalisation with the grouped-query repeat, and
// the gated RMSNorm.
//
//   ssm_a       ssm_a = -exp(A_log), the per-head factor of the gate, which
//               both Foundry pages prepare once on the host
//               (ssm_gated_delta.cu fc_ssm_decay_gate comment)
//   decay gate  g = ssm_a * softplus(a + dt_bias), softplus guarded at 20
//               (ssm_gated_delta.cu fc_ssm_decay_gate / _nx; fm_kernel_ssm.m
//               "Decay gate")
//   sigmoid     beta = 1 / (1 + exp(-b))          (ssm_gated_delta.cu fc_sigmoid)
//   L2 + GQA    x / max(||x||, eps) per K-head; V-head vh reads K-head
//               vh mod HK (ssm_gated_delta.cu fc_ssm_qknorm_gqa; mlx-native
//               "GQA: tiled mapping")
//   gated norm  y / sqrt(mean(y^2) + eps) * w * silu(z), w shared by all heads
//               (fm_kernel_ssm.m "Gated RMSNorm"; ssm_gated_delta.cu Kernel 3)
//
// The row kernels give one wave to a row; each lane reads float4 slots
// 4*(lane + 64*m) of it, and the row's sum of squares is a wave-wide DPP /
// swizzle / bpermute reduction with no LDS array and no barrier.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

__global__ __launch_bounds__(256) void decay_gate_kernel(const float* __restrict__ a,
                                                         const float* __restrict__ dt_bias,
                                                         const float* __restrict__ ssm_a,
                                                         float* __restrict__ g, int n_heads,
                                                         int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int h = (int)(idx % n_heads);
  g[idx] = decay_gate(a[idx], dt_bias[h], ssm_a[h]);
}

__global__ __launch_bounds__(256) void ssm_a_kernel(const float* __restrict__ A_log,
                                                    float* __restrict__ out, int n) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  out[idx] = ssm_a_of(A_log[idx]);
}

__global__ __launch_bounds__(256) void sigmoid_kernel(const float* x, float* y, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  y[idx] = sigmoid(x[idx]);
}

#pragma clang fp contract(off)
__global__ __launch_bounds__(256) void l2norm_gqa_kernel(const float* __restrict__ x,
                                                         float* __restrict__ out, int64_t n_groups,
                                                         int n_k_heads, int n_v_heads,
                                                         int head_dim, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t grp = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (grp >= n_groups) return;  // uniform across the wave
  const int64_t r = grp / n_k_heads;
  const int kh = (int)(grp % n_k_heads);
  const int d4 = head_dim >> 2;
  const float* src = x + grp * head_dim;
  const float ss = row_sumsq(src, d4, lane);
  const float inv = inv_l2norm(ss, eps);
  for (int m = lane; m < d4; m += 64) {
    float4 v = load4(src + 4 * m);
    v.x = v.x * inv;
    v.y = v.y * inv;
    v.z = v.z * inv;
    v.w = v.w * inv;
    for (int vh = kh; vh < n_v_heads; vh += n_k_heads)
      store4(out + (r * n_v_heads + vh) * head_dim + 4 * m, v);
  }
}

__device__ __forceinline__ float4 load_z4(const float* z) { return load4(z); }

__device__ __forceinline__ float4 load_z4(const uint16_t* z) {
  const uint2 b = *reinterpret_cast<const uint2*>(z);
  return make_float4(bf16_to_float((uint16_t)(b.x & 0xFFFFu)), bf16_to_float((uint16_t)(b.x >> 16)),
                     bf16_to_float((uint16_t)(b.y & 0xFFFFu)), bf16_to_float((uint16_t)(b.y >> 16)));
}

// ZT is float, or uint16_t for a bf16 gate z (widened exactly on load).
template <typename ZT>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const float* __restrict__ y,
                                                            const float* __restrict__ w,
                                                            const ZT* __restrict__ z,
                                                            float* __restrict__ out,
                                                            int64_t n_rows, int head_dim,
                                                            float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // uniform across the wave
  const int d4 = head_dim >> 2;
  const float* yr = y + row * head_dim;
  const ZT* zr = z + row * head_dim;
  float* orow = out + row * head_dim;
  const float ss = row_sumsq(yr, d4, lane);
  const float inv = 1.0f / sqrtf(ss / (float)head_dim + eps);
  for (int m = lane; m < d4; m += 64) {
    const float4 yv = load4(yr + 4 * m);
    const float4 zv = load_z4(zr + 4 * m);
    const float4 wv = load4(w + 4 * m);
    float4 o;
    o.x = yv.x * inv * wv.x * silu(zv.x);
    o.y = yv.y * inv * wv.y * silu(zv.y);
    o.z = yv.z * inv * wv.z * silu(zv.z);
    o.w = yv.w * inv * wv.w * silu(zv.w);
    store4(orow + 4 * m, o);
  }
}

// The same norm for head_dim = 128, the workloads' size: a half-wave per row
// (one float4 per lane), two rows per wave at a time and kNormIters pairs per
// wave, with every load issued before any arithmetic. The sum of squares is
// the per-lane FMA chain of row_sumsq followed by the first five butterfly
// steps of group_sum<64>; in row_sumsq the other 32 lanes contribute exact
// zeros to the sixth step, so the result is the same bit for bit.
constexpr int kNormIters = 2;

template <typename ZT>
__global__ __launch_bounds__(256) void gated_rmsnorm_d128_kernel(
    const float* __restrict__ y, const float* __restrict__ w, const ZT* __restrict__ z,
    float* __restrict__ out, int64_t n_rows, float eps) {
  constexpr int D = 128;
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  float4 yv[kNormIters], zv[kNormIters];
  int64_t rows[kNormIters];
#pragma unroll
  for (int it = 0; it < kNormIters; ++it) {
    rows[it] = (wave * kNormIters + it) * 2 + half;
    const int64_t r = rows[it] < n_rows ? rows[it] : n_rows - 1;   // rows past the end: not stored
    yv[it] = load4_stream(y + r * D + 4 * l32);
    zv[it] = load_z4(z + r * D + 4 * l32);
  }
  const float4 wv = load4(w + 4 * l32);
#pragma unroll
  for (int it = 0; it < kNormIters; ++it) {
    float ss = 0.0f;
    ss = __builtin_fmaf(yv[it].x, yv[it].x, ss);
    ss = __builtin_fmaf(yv[it].y, yv[it].y, ss);
    ss = __builtin_fmaf(yv[it].z, yv[it].z, ss);
    ss = __builtin_fmaf(yv[it].w, yv[it].w, ss);
    ss = group_sum<32>(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
    float4 o;
    o.x = yv[it].x * inv * wv.x * silu(zv[it].x);
    o.y = yv[it].y * inv * wv.y * silu(zv[it].y);
    o.z = yv[it].z * inv * wv.z * silu(zv[it].z);
    o.w = yv[it].w * inv * wv.w * silu(zv[it].w);
    if (rows[it] < n_rows) store4(out + rows[it] * D + 4 * l32, o);
  }
}
#pragma clang fp contract(fast)

template <typename ZT>
int launch_gated_rmsnorm(const float* y, const float* w, const ZT* z, float* out, int64_t n_rows,
                         int head_dim, float eps, hipStream_t s) {
  if (head_dim == 128) {
    const int64_t rows_per_block = 4 * 2 * kNormIters;
    return launch(gated_rmsnorm_d128_kernel<ZT>, dim3(grid_for(n_rows, rows_per_block)),
                  dim3(256), 0, s, y, w, z, out, n_rows, eps);
  }
  return launch(gated_rmsnorm_kernel<ZT>, dim3(grid_for(n_rows, 4)), dim3(256), 0, s, y, w, z, out,
                n_rows, head_dim, eps);
}

}  // namespace gdn

using namespace gdn;

extern "C" int gdn_ssm_a(const float* A_log, float* ssm_a, int n_heads, void* stream) {
  if (n_heads < 0) return GDN_ESIZE;
  if (n_heads == 0) return GDN_OK;
  if (!A_log || !ssm_a) return GDN_ENULL;
  return launch(ssm_a_kernel, dim3(grid_for(n_heads, 256)), dim3(256), 0, as_stream(stream),
                A_log, ssm_a, n_heads);
}

extern "C" int gdn_decay_gate(const float* a, const float* dt_bias, const float* ssm_a, float* g,
                              int n_heads, int64_t rows, void* stream) {
  int64_t total;
  if (n_heads <= 0 || rows < 0 || !mul_ok(rows, n_heads, &total)) return GDN_ESIZE;
  if (rows == 0) return GDN_OK;
  if (!a || !dt_bias || !ssm_a || !g) return GDN_ENULL;
  if (total / 256 >= (int64_t(1) << 31)) return GDN_ESIZE;
  return launch(decay_gate_kernel, dim3(grid_for(total, 256)), dim3(256), 0, as_stream(stream), a,
                dt_bias, ssm_a, g, n_heads, total);
}

extern "C" int gdn_sigmoid(const float* x, float* y, int64_t n, void* stream) {
  if (n < 0 || n > kMaxElems || n / 256 >= (int64_t(1) << 31)) return GDN_ESIZE;
  if (n == 0) return GDN_OK;
  if (!x || !y) return GDN_ENULL;
  return launch(sigmoid_kernel, dim3(grid_for(n, 256)), dim3(256), 0, as_stream(stream), x, y, n);
}

extern "C" int gdn_l2norm_gqa(const float* x, float* out, int64_t rows, int n_k_heads,
                              int n_v_heads, int head_dim, float eps, void* stream) {
  if (rows < 0 || n_k_heads <= 0 || n_v_heads <= 0 || head_dim <= 0) return GDN_ESIZE;
  if (n_v_heads % n_k_heads != 0) return GDN_ESIZE;
  if (head_dim % 4 != 0 || head_dim > 1024) return GDN_EUNSUPPORTED;
  if (rows == 0) return GDN_OK;
  if (!x || !out) return GDN_ENULL;
  int64_t groups, elems;
  if (!mul_ok(rows, n_k_heads, &groups) || !mul_ok(rows * n_v_heads, head_dim, &elems))
    return GDN_ESIZE;
  if (groups / 4 >= (int64_t(1) << 31)) return GDN_ESIZE;
  if (!aligned16(x) || !aligned16(out)) return GDN_EALIGN;
  return launch(l2norm_gqa_kernel, dim3(grid_for(groups, 4)), dim3(256), 0, as_stream(stream), x,
                out, groups, n_k_heads, n_v_heads, head_dim, eps);
}

extern "C" int gdn_gated_rmsnorm(const float* y, const float* w, const float* z, float* out,
                                 int64_t n_rows, int head_dim, float eps, void* stream) {
  int64_t elems;
  if (n_rows < 0 || head_dim <= 0 || !mul_ok(n_rows, head_dim, &elems)) return GDN_ESIZE;
  if (head_dim % 4 != 0 || head_dim > 1024) return GDN_EUNSUPPORTED;
  if (n_rows == 0) return GDN_OK;
  if (!y || !w || !z || !out) return GDN_ENULL;
  if (n_rows / 4 >= (int64_t(1) << 31)) return GDN_ESIZE;
  if (!aligned16(y) || !aligned16(w) || !aligned16(z) || !aligned16(out)) return GDN_EALIGN;
  return launch_gated_rmsnorm<float>(y, w, z, out, n_rows, head_dim, eps, as_stream(stream));
}

namespace gdn {
int launch_gated_rmsnorm_bf16z(const float* y, const float* w, const uint16_t* z, float* out,
                               int64_t n_rows, int head_dim, float eps, hipStream_t s) {
  return launch_gated_rmsnorm<uint16_t>(y, w, z, out, n_rows, head_dim, eps, s);
}
}  // namespace gdn
