// Measurement probes of the benchmark: the fp32 FMA issue rate of the chip as
// libgdn.so is built (packed FP32 disabled), and the issue rate of the matrix
// instructions the chunked scan uses. Not steps of the method, and built into
// their own library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_probe.h"

namespace {

constexpr int kProbeChains = 16;

__global__ __launch_bounds__(256) void probe_fma_kernel(float* __restrict__ out, int iters,
                                                        float a, float b) {
  float c[kProbeChains];
#pragma unroll
  for (int i = 0; i < kProbeChains; ++i) c[i] = (float)(threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kProbeChains; ++i) c[i] = __builtin_fmaf(c[i], a, b);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kProbeChains; ++i) s += c[i];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// NCH independent accumulator chains of v_mfma_f32_16x16x4f32 per wave.
template <int NCH>
__global__ __launch_bounds__(256) void probe_mfma_f32_kernel(float* __restrict__ out, int iters,
                                                             float a, float b) {
  f32x4 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, (float)c};
  const float av = a + threadIdx.x * 1e-6f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// NCH independent accumulator chains of v_mfma_f32_16x16x32_bf16 per wave.
template <int NCH>
__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(float* __restrict__ out, int iters,
                                                              float a, float b) {
  f32x4 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, (float)c};
  bf16x8 av, bv;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    av[i] = (__bf16)(a + i * 1e-3f + threadIdx.x * 1e-6f);
    bv[i] = (__bf16)(b + i * 1e-3f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

int launch_status(hipError_t e) { return e == hipSuccess ? 0 : 5; }

}  // namespace

extern "C" int gdn_probe_fma(float* out, int n_blocks, int iters, float a, float b,
                             void* stream) {
  if (n_blocks <= 0 || iters <= 0 || n_blocks > (1 << 20)) return 2;
  if (!out) return 1;
  void* args[] = {&out, &iters, &a, &b};
  return launch_status(hipLaunchKernel(reinterpret_cast<const void*>(probe_fma_kernel),
                                       dim3((unsigned)n_blocks), dim3(256), args, 0,
                                       reinterpret_cast<hipStream_t>(stream)));
}

extern "C" int gdn_probe_mfma(int kind, int chains, float* out, int n_blocks, int iters,
                              void* stream) {
  if (n_blocks <= 0 || iters <= 0 || n_blocks > (1 << 20)) return 2;
  if (!(kind == 0 || kind == 1) || !(chains == 1 || chains == 2 || chains == 4)) return 3;
  if (!out) return 1;
  float a = 0.999f, b = 1e-3f;
  void* args[] = {&out, &iters, &a, &b};
  const void* k = nullptr;
  if (kind == 0)
    k = chains == 1 ? reinterpret_cast<const void*>(probe_mfma_f32_kernel<1>)
        : chains == 2 ? reinterpret_cast<const void*>(probe_mfma_f32_kernel<2>)
                      : reinterpret_cast<const void*>(probe_mfma_f32_kernel<4>);
  else
    k = chains == 1 ? reinterpret_cast<const void*>(probe_mfma_bf16_kernel<1>)
        : chains == 2 ? reinterpret_cast<const void*>(probe_mfma_bf16_kernel<2>)
                      : reinterpret_cast<const void*>(probe_mfma_bf16_kernel<4>);
  return launch_status(hipLaunchKernel(k, dim3((unsigned)n_blocks), dim3(256), args, 0,
                                       reinterpret_cast<hipStream_t>(stream)));
}
