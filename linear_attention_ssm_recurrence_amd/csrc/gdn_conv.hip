// Causal depthwise conv1d + SiLU on gfx950, one step (decode) and over many
// positions (scan).
//
// Per channel c the window is the K-1 stored inputs (oldest first) followed by
// the current input; the sum starts from the newest tap, x * w[c][K-1], then
// adds history[u] * w[c][u] in ascending u, and the output is SiLU of the sum.
// The history then drops its oldest entry and appends the raw input (Foundry
// fm_kernel_ssm.m "Causal depthwise conv1d + SiLU"; ssm_gated_delta.cu
// Kernel 2 and fc_ssm_conv1d_silu_seq).
//
// The history is nothing but the last K-1 raw inputs, so no output depends on
// an earlier output: the scan is data-parallel over positions as well as over
// channels. Each thread takes one channel (four consecutive channels when
// conv_dim is a multiple of 4, the buffers are 16-byte aligned and there are
// more than 8 positions, so that every access is a 16-byte vector) and a
// chunk of positions, reading K-1 inputs before its chunk as a halo (from
// conv_state for positions before the first). Every kernel evaluates each
// position with the same conv_point, so the scans and single steps agree bit
// for bit.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// Positions per thread of the four-channel scan. Measured at 1 x 4096 x 8192
// (K = 4) with the input cold (four input/output sets in rotation, 1 GiB,
// beyond the last-level cache): 8 positions 44.4-45.3 us per launch, 12
// 45.6, 16 49.0, 4 53.5; the per-channel scan 49.4-51.4 us with ordinary
// access and 46.2-46.8 us with non-temporal access.
constexpr int kConvTB4 = 8;

template <int K>
__global__ __launch_bounds__(256) void conv_step_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        float* __restrict__ conv_state,
                                                        float* __restrict__ out, int64_t total,
                                                        int conv_dim) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // n * C + c
  if (idx >= total) return;
  const int c = (int)(idx % conv_dim);
  float wc[K], hist[K - 1];
#pragma unroll
  for (int u = 0; u < K; ++u) wc[u] = w[(int64_t)c * K + u];
  float* cs = conv_state + idx * (K - 1);
#pragma unroll
  for (int u = 0; u < K - 1; ++u) hist[u] = cs[u];
  const float xv = x[idx];
  out[idx] = conv_point<K>(xv, hist, wc);
#pragma unroll
  for (int u = 0; u + 1 < K - 1; ++u) cs[u] = hist[u + 1];
  cs[K - 2] = xv;
}

// Scan: block (cb, chunk, n) covers channels cb*256 .. +255 and positions
// chunk*TB .. +TB-1 of sequence n. With SNAP the history after every position
// t is also written to snaps[N][T][C][K-1] (the conv_state layout, one image
// per position), for speculative decoding's partial accept (ssm_gated_delta.cu
// fc_ssm_conv1d_silu_seq, "snaps").
template <int K, int TB, bool SNAP>
__global__ __launch_bounds__(256) void conv_scan_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        float* __restrict__ conv_state,
                                                        float* __restrict__ out,
                                                        float* __restrict__ snaps, int n_tokens,
                                                        int conv_dim, int c_blocks,
                                                        int t_chunks) {
  const int cb = blockIdx.x % c_blocks;
  const int chunk = (blockIdx.x / c_blocks) % t_chunks;
  const int64_t n = blockIdx.x / ((int64_t)c_blocks * t_chunks);
  const int c = cb * 256 + threadIdx.x;
  if (c >= conv_dim) return;
  const int t0 = chunk * TB;
  const float* xc = x + n * (int64_t)n_tokens * conv_dim + c;
  float* oc = out + n * (int64_t)n_tokens * conv_dim + c;
  float* cs = conv_state + (n * conv_dim + c) * (K - 1);

  float wc[K];
#pragma unroll
  for (int u = 0; u < K; ++u) wc[u] = w[(int64_t)c * K + u];

  // hist = inputs at positions t0-K+1 .. t0-1 (negative positions: conv_state)
  float hist[K - 1];
#pragma unroll
  for (int u = 0; u < K - 1; ++u) {
    const int t = t0 - (K - 1) + u;
    hist[u] = t < 0 ? cs[K - 1 + t] : xc[(int64_t)t * conv_dim];
  }
  // The chunk-0 thread is the only reader of the old conv_state, so it also
  // writes the new one: the last K-1 entries of (old history ++ inputs).
  float fin[K - 1];
  if (chunk == 0) {
#pragma unroll
    for (int u = 0; u < K - 1; ++u) {
      const int t = n_tokens - (K - 1) + u;
      fin[u] = t < 0 ? cs[K - 1 + t] : xc[(int64_t)t * conv_dim];
    }
  }
  // every input of the chunk loaded before any arithmetic, so the loads are
  // in flight together (positions past the end read the last one, unused);
  // inputs and outputs are touched once per launch: non-temporal
  float xs[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const int t = t0 + i < n_tokens ? t0 + i : n_tokens - 1;
    xs[i] = __builtin_nontemporal_load(xc + (int64_t)t * conv_dim);
  }
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const int t = t0 + i;
    if (t < n_tokens)
      __builtin_nontemporal_store(conv_point<K>(xs[i], hist, wc), oc + (int64_t)t * conv_dim);
#pragma unroll
    for (int u = 0; u + 1 < K - 1; ++u) hist[u] = hist[u + 1];
    hist[K - 2] = xs[i];
    if constexpr (SNAP) {
      if (t < n_tokens) {
        float* sn = snaps + ((n * n_tokens + t) * conv_dim + c) * (K - 1);
#pragma unroll
        for (int u = 0; u < K - 1; ++u) sn[u] = hist[u];
      }
    }
  }
  if (chunk == 0) {
#pragma unroll
    for (int u = 0; u < K - 1; ++u) cs[u] = fin[u];
  }
}

// The same scan with four consecutive channels per thread (conv_dim a
// multiple of 4, every pointer 16-byte aligned, more than TB positions, so
// that a sequence spans at least two chunks): each input and output row
// piece is one float4, and a channel group's weights, history and history
// snapshots (4 (K-1) or 4 K consecutive floats) are whole float4s. Each
// channel goes through the same conv_point in the same order as in
// conv_scan_kernel, so the two kernels, and single steps, agree bit for bit.
template <int K, int TB, bool SNAP>
__global__ __launch_bounds__(256) void conv_scan4_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ w,
                                                         float* __restrict__ conv_state,
                                                         float* __restrict__ out,
                                                         float* __restrict__ snaps, int n_tokens,
                                                         int conv_dim, int c_blocks,
                                                         int t_chunks) {
  constexpr int H1 = K - 1;
  const int cb = blockIdx.x % c_blocks;
  const int chunk = (blockIdx.x / c_blocks) % t_chunks;
  const int64_t n = blockIdx.x / ((int64_t)c_blocks * t_chunks);
  const int c = (cb * 256 + (int)threadIdx.x) * 4;   // channels c .. c+3
  if (c >= conv_dim) return;
  const int t0 = chunk * TB;
  const float* xc = x + n * (int64_t)n_tokens * conv_dim + c;
  float* oc = out + n * (int64_t)n_tokens * conv_dim + c;
  float* cs = conv_state + (n * conv_dim + c) * H1;   // 4 (K-1) floats, channel-major

  float wf[4 * K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const float4 v = load4(w + (int64_t)c * K + 4 * i);
    wf[4 * i] = v.x, wf[4 * i + 1] = v.y, wf[4 * i + 2] = v.z, wf[4 * i + 3] = v.w;
  }
  float wc[4][K];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int u = 0; u < K; ++u) wc[j][u] = wf[j * K + u];

  // the old history, read by the chunk-0 threads only
  float old[4 * H1];
  if (chunk == 0) {
#pragma unroll
    for (int i = 0; i < H1; ++i) {
      const float4 v = load4(cs + 4 * i);
      old[4 * i] = v.x, old[4 * i + 1] = v.y, old[4 * i + 2] = v.z, old[4 * i + 3] = v.w;
    }
  }
  // hist = inputs at positions t0-K+1 .. t0-1 (negative positions: the old history)
  float hist[4][H1];
#pragma unroll
  for (int u = 0; u < H1; ++u) {
    const int t = t0 - H1 + u;
    float4 v;
    if (t < 0) v = make_float4(old[H1 + t], old[H1 + H1 + t], old[2 * H1 + H1 + t],
                               old[3 * H1 + H1 + t]);
    else v = load4(xc + (int64_t)t * conv_dim);
    hist[0][u] = v.x, hist[1][u] = v.y, hist[2][u] = v.z, hist[3][u] = v.w;
  }
  // The chunk-0 thread is the only reader of the old history, so it also
  // writes the new one: the last K-1 entries of (old history ++ inputs).
  float fin[4][H1];
  if (chunk == 0) {
#pragma unroll
    for (int u = 0; u < H1; ++u) {
      const int t = n_tokens - H1 + u;
      float4 v;
      if (t < 0) v = make_float4(old[H1 + t], old[H1 + H1 + t], old[2 * H1 + H1 + t],
                                 old[3 * H1 + H1 + t]);
      else v = load4(xc + (int64_t)t * conv_dim);
      fin[0][u] = v.x, fin[1][u] = v.y, fin[2][u] = v.z, fin[3][u] = v.w;
    }
  }
  // every input of the chunk loaded before any arithmetic (positions past
  // the end read the last one, unused)
  float4 xs[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const int t = t0 + i < n_tokens ? t0 + i : n_tokens - 1;
    // non-temporal except the last K-1 positions, which the next chunk's
    // thread reads again as its halo
    xs[i] = (i >= TB - H1) ? load4(xc + (int64_t)t * conv_dim)
                           : load4_stream(xc + (int64_t)t * conv_dim);
  }
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const int t = t0 + i;
    const float xv[4] = {xs[i].x, xs[i].y, xs[i].z, xs[i].w};
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = conv_point<K>(xv[j], hist[j], wc[j]);
#pragma unroll
      for (int u = 0; u + 1 < H1; ++u) hist[j][u] = hist[j][u + 1];
      hist[j][H1 - 1] = xv[j];
    }
    if (t < n_tokens)   // written once per launch: non-temporal
      store4_stream(oc + (int64_t)t * conv_dim, make_float4(o[0], o[1], o[2], o[3]));
    if constexpr (SNAP) {
      if (t < n_tokens) {
        float sf[4 * H1];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int u = 0; u < H1; ++u) sf[j * H1 + u] = hist[j][u];
        float* sn = snaps + ((n * n_tokens + t) * conv_dim + c) * H1;
#pragma unroll
        for (int q4 = 0; q4 < H1; ++q4)
          store4(sn + 4 * q4, make_float4(sf[4 * q4], sf[4 * q4 + 1], sf[4 * q4 + 2], sf[4 * q4 + 3]));
      }
    }
  }
  if (chunk == 0) {
    float sf[4 * H1];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < H1; ++u) sf[j * H1 + u] = fin[j][u];
#pragma unroll
    for (int q4 = 0; q4 < H1; ++q4)
      store4(cs + 4 * q4, make_float4(sf[4 * q4], sf[4 * q4 + 1], sf[4 * q4 + 2], sf[4 * q4 + 3]));
  }
}

static int check_conv(const float* x, const float* w, float* conv_state, float* out, int n_seqs,
                      int n_tokens, int conv_dim, int conv_kernel) {
  if (n_seqs < 0 || n_tokens < 0 || conv_dim <= 0 || conv_kernel <= 0) return GDN_ESIZE;
  if (conv_kernel < 2 || conv_kernel > 4) return GDN_EUNSUPPORTED;
  if (n_seqs == 0 || n_tokens == 0) return kNothingToDo;
  if (!x || !w || !conv_state || !out) return GDN_ENULL;
  int64_t a, b;
  if (!mul_ok(n_seqs, n_tokens, &a) || !mul_ok(a, conv_dim, &b)) return GDN_ESIZE;
  if (!mul_ok((int64_t)n_seqs * conv_dim, conv_kernel, &a)) return GDN_ESIZE;
  return GDN_OK;
}

template <int K>
static int launch_conv_step(const float* x, const float* w, float* cs, float* out, int n_seqs,
                            int conv_dim, hipStream_t s) {
  const int64_t total = (int64_t)n_seqs * conv_dim;
  if (grid_for(total, 256) == 0 || total / 256 >= (int64_t(1) << 31)) return GDN_ESIZE;
  return launch(conv_step_kernel<K>, dim3(grid_for(total, 256)), dim3(256), 0, s, x, w, cs, out,
                total, conv_dim);
}

template <int K>
static int launch_conv_scan(const float* x, const float* w, float* cs, float* out, float* snaps,
                            int n_seqs, int n_tokens, int conv_dim, hipStream_t s) {
  // With one chunk of positions or fewer (a speculative verify of a few
  // tokens) the four-channel scan would run a quarter of the threads in a
  // single round of waves: the per-channel scan hides the memory latency
  // better there (measured at 64 x 4 x 8192 with snapshots).
  if (n_tokens > kConvTB4 && conv_dim % 4 == 0 && aligned16(x) && aligned16(w) &&
      aligned16(cs) && aligned16(out) && (!snaps || aligned16(snaps))) {
    constexpr int TB4 = kConvTB4;
    const int c_blocks = (conv_dim / 4 + 255) / 256;
    const int t_chunks = (n_tokens + TB4 - 1) / TB4;
    const int64_t blocks = (int64_t)n_seqs * c_blocks * t_chunks;
    if (blocks >= (int64_t(1) << 31)) return GDN_ESIZE;
    if (snaps)
      return launch(conv_scan4_kernel<K, TB4, true>, dim3((unsigned)blocks), dim3(256), 0, s, x,
                    w, cs, out, snaps, n_tokens, conv_dim, c_blocks, t_chunks);
    return launch(conv_scan4_kernel<K, TB4, false>, dim3((unsigned)blocks), dim3(256), 0, s, x,
                  w, cs, out, nullptr, n_tokens, conv_dim, c_blocks, t_chunks);
  }
  constexpr int TB = 16;
  const int c_blocks = (conv_dim + 255) / 256;
  const int t_chunks = (n_tokens + TB - 1) / TB;
  const int64_t blocks = (int64_t)n_seqs * c_blocks * t_chunks;
  if (blocks >= (int64_t(1) << 31)) return GDN_ESIZE;
  if (snaps)
    return launch(conv_scan_kernel<K, TB, true>, dim3((unsigned)blocks), dim3(256), 0, s, x, w,
                  cs, out, snaps, n_tokens, conv_dim, c_blocks, t_chunks);
  return launch(conv_scan_kernel<K, TB, false>, dim3((unsigned)blocks), dim3(256), 0, s, x, w, cs,
                out, nullptr, n_tokens, conv_dim, c_blocks, t_chunks);
}

}  // namespace gdn

using namespace gdn;

extern "C" int gdn_conv1d_silu(const float* x, const float* w, float* conv_state, float* out,
                               int n_seqs, int conv_dim, int conv_kernel, void* stream) {
  const int rc = check_conv(x, w, conv_state, out, n_seqs, 1, conv_dim, conv_kernel);
  if (rc != GDN_OK) return finish_check(rc);
  hipStream_t s = as_stream(stream);
  switch (conv_kernel) {
    case 2: return launch_conv_step<2>(x, w, conv_state, out, n_seqs, conv_dim, s);
    case 3: return launch_conv_step<3>(x, w, conv_state, out, n_seqs, conv_dim, s);
    case 4: return launch_conv_step<4>(x, w, conv_state, out, n_seqs, conv_dim, s);
  }
  return GDN_EUNSUPPORTED;
}

static int conv_seq(const float* x, const float* w, float* conv_state, float* out, float* snaps,
                    int n_seqs, int n_tokens, int conv_dim, int conv_kernel, hipStream_t s) {
  switch (conv_kernel) {
    case 2: return launch_conv_scan<2>(x, w, conv_state, out, snaps, n_seqs, n_tokens, conv_dim, s);
    case 3: return launch_conv_scan<3>(x, w, conv_state, out, snaps, n_seqs, n_tokens, conv_dim, s);
    case 4: return launch_conv_scan<4>(x, w, conv_state, out, snaps, n_seqs, n_tokens, conv_dim, s);
  }
  return GDN_EUNSUPPORTED;
}

extern "C" int gdn_conv1d_silu_seq(const float* x, const float* w, float* conv_state, float* out,
                                   int n_seqs, int n_tokens, int conv_dim, int conv_kernel,
                                   void* stream) {
  const int rc = check_conv(x, w, conv_state, out, n_seqs, n_tokens, conv_dim, conv_kernel);
  if (rc != GDN_OK) return finish_check(rc);
  return conv_seq(x, w, conv_state, out, nullptr, n_seqs, n_tokens, conv_dim, conv_kernel,
                  as_stream(stream));
}

extern "C" int gdn_conv1d_silu_seq_ex(const float* x, const float* w, float* conv_state,
                                      float* out, float* snaps, int n_seqs, int n_tokens,
                                      int conv_dim, int conv_kernel, void* stream) {
  const int rc = check_conv(x, w, conv_state, out, n_seqs, n_tokens, conv_dim, conv_kernel);
  if (rc != GDN_OK) return finish_check(rc);
  int64_t e;
  if (snaps && !mul_ok((int64_t)n_seqs * n_tokens * conv_dim, conv_kernel - 1, &e)) return GDN_ESIZE;
  return conv_seq(x, w, conv_state, out, snaps, n_seqs, n_tokens, conv_dim, conv_kernel,
                  as_stream(stream));
}
