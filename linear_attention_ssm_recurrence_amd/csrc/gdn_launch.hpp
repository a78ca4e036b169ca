// Host-side helpers shared by the C-ABI entry points: argument checks and the
// launch error check. Every entry point validates all of its arguments before
// it enqueues anything, so a non-zero return means nothing was launched.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gdn.h"

namespace gdn {

// Internal result of an argument check: valid, but there is no work (a zero
// count). The entry point returns GDN_OK without launching anything.
constexpr int kNothingToDo = -1;

inline int finish_check(int rc) { return rc == kNothingToDo ? GDN_OK : rc; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool is_state_size(int s) { return s == 32 || s == 64 || s == 128 || s == 256; }

// Largest element count any single array may have: keeps every flattened
// index inside int64 with room, and every grid inside the launch limits.
constexpr int64_t kMaxElems = int64_t(1) << 40;

inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxElems / a) return false;
  *out = a * b;
  return true;
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ELAUNCH;
}

inline unsigned grid_for(int64_t items, int per_block) {
  return (unsigned)((items + per_block - 1) / per_block);
}

// Compute units of the current device (queried once per device; 256 on
// MI355X). Used only to choose between launch shapes, never for correctness.
// The cache is atomic, so host threads that call the library concurrently
// may each query it, but never read a torn value.
inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The dispatcher hands workgroup b to XCD b % 8. This maps a block id to a
// logical block so that consecutive logical blocks share an XCD (and its L2),
// when the grid divides evenly.
constexpr int kXcds = 8;

__device__ __forceinline__ unsigned xcd_group(unsigned bid, unsigned nblocks) {
  if (nblocks % kXcds != 0) return bid;
  return (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
}

// Internal launchers shared between translation units (no argument checks:
// the calling entry point has validated everything).
int launch_gated_rmsnorm_bf16z(const float* y, const float* w, const uint16_t* z, float* out,
                               int64_t n_rows, int head_dim, float eps, hipStream_t s);

}  // namespace gdn
