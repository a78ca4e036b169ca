// Measurement probe: the fp32 FMA issue rate of the chip as this library is
// built (packed FP32 disabled). Not a step of the method.
#include "gdn_launch.hpp"
#include "gdn_probe.h"

namespace gdn {

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

}  // namespace gdn

extern "C" int gdn_probe_fma(float* out, int n_blocks, int iters, float a, float b,
                             void* stream) {
  if (n_blocks <= 0 || iters <= 0 || n_blocks > (1 << 20)) return GDN_ESIZE;
  if (!out) return GDN_ENULL;
  hipLaunchKernelGGL(gdn::probe_fma_kernel, dim3((unsigned)n_blocks), dim3(256), 0,
                     gdn::as_stream(stream), out, iters, a, b);
  return gdn::launch_status();
}
