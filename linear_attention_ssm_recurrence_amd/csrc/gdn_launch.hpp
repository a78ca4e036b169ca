// Host-side helpers shared by the C-ABI entry points: argument checks and the
// launch error check. Every entry point validates all of its arguments before
// it enqueues anything, so a non-zero return means nothing was launched.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <tuple>
#include <utility>

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

// Enqueues kernel<<<grid, block, shmem, s>>>(args...) and returns the status
// of this launch alone: hipLaunchKernel's own return value. (hipGetLastError
// would also report, and clear, an error left pending on the calling thread
// by an earlier, unrelated call, and so could call a launch that was enqueued
// a failure.) Each argument is converted to the kernel's parameter type.
template <typename... P, size_t... I>
inline int launch_with(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                       std::tuple<P...>& vals, std::index_sequence<I...>) {
  void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1] = {static_cast<void*>(&std::get<I>(vals))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, s) ==
                 hipSuccess
             ? GDN_OK
             : GDN_ELAUNCH;
}

template <typename... P, typename... A>
inline int launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                  A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "a kernel argument is missing or extra");
  std::tuple<P...> vals(static_cast<P>(args)...);
  return launch_with(kernel, grid, block, shmem, s, vals, std::index_sequence_for<P...>{});
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

// Size checks of the scan kernels, for shapes the caller has already found
// valid: GDN_OK, or GDN_ESIZE when an array or a grid would be too large.
int recurrence_size_check(int64_t n_seqs, int64_t n_tokens, int n_v_heads, int state_size);
int chunked_size_check(int64_t n_seqs, int64_t n_tokens, int n_v_heads);

// Internal launchers shared between translation units (no argument checks:
// the calling entry point has validated everything).
int launch_gated_rmsnorm_bf16z(const float* y, const float* w, const uint16_t* z, float* out,
                               int64_t n_rows, int head_dim, float eps, hipStream_t s);

}  // namespace gdn
