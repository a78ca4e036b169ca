// Measurement probe of the benchmark: the fp32 FMA issue rate of the chip as
// libgdn.so is built (packed FP32 disabled). Not a step of the method, and
// built into its own library.
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

}  // namespace

extern "C" int gdn_probe_fma(float* out, int n_blocks, int iters, float a, float b,
                             void* stream) {
  if (n_blocks <= 0 || iters <= 0 || n_blocks > (1 << 20)) return 2;
  if (!out) return 1;
  void* args[] = {&out, &iters, &a, &b};
  return hipLaunchKernel(reinterpret_cast<const void*>(probe_fma_kernel), dim3((unsigned)n_blocks),
                         dim3(256), args, 0, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? 0
             : 5;
}
