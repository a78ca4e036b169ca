// Chained prefill of one layer of the Gated DeltaNet block on gfx950: bf16
// activations over n_tokens positions, fp32 state.
//
// The per-token decode order of ssm_gated_delta.cu's batched ("_nx" / "_seq")
// kernels, chained: conv1d + SiLU over the positions, L2 norm of q and k per
// K-head, v passed through, decay gate and sigmoid per position, the
// sequential scan (V-head h reading K-head h mod HK), then the gated RMSNorm.
// Three stages:
//   1. prefill_frontend_kernel: conv + L2 norm + gate + sigmoid, fused;
//   2. the scan on its outputs: the sequential scan of gdn_recurrence_seq_ex,
//      or the chunked one of gdn_recurrence_seq_chunked (GDN_SCAN_CHUNKED);
//   3. the gated RMSNorm with the bf16 gate z.
// The intermediates (normalised q and k per K-head, v, g, beta, y, and the
// chunked scan's workspace) live in a caller-provided workspace.
//
// Front end. A wave owns one "head part" (the S = 128 channels of q or k of a
// K-head, or of v of a V-head) of one sequence over TB = 32 positions: lanes
// 0-31 take the first 16 positions, lanes 32-63 the next 16, each lane four
// consecutive channels with its conv window in registers. The L2 norm of a
// position is a 32-lane DPP sum. The positions of a wave are a contiguous
// range, so every output of a position depends only on the K-1 raw inputs
// before it: the positions are independent, and only the lanes that own
// position 0 read the old conv history, which is why they (and nobody else)
// write the new one.
//
// Every value goes through the same device function and reduction order as in
// the fused decode layer (gdn_block.hip), so with the sequential scan a
// prefill over T positions equals T calls of gdn_decode_block_bf16 bit for
// bit; the chunked scan agrees with them within the fp32 tolerance.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kPrefillS = 128;
constexpr int kPrefillTH = 16;               // positions per half-wave
constexpr int kPrefillTB = 2 * kPrefillTH;   // positions per wave
constexpr int kPrefillWaves = 4;             // head parts per block

struct PrefillWorkspace {
  float *q, *k, *v, *g, *beta, *y;
  void* chunk;          // workspace of the chunked scan
  size_t chunk_bytes;
};

inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Carves the workspace (or only sizes it when base is null).
inline size_t prefill_layout(int64_t N, int64_t T, int64_t HK, int64_t H, int64_t S, char* base,
                             PrefillWorkspace* ws) {
  size_t off = 0;
  auto take = [&](int64_t elems, float** p) {
    if (base) *p = reinterpret_cast<float*>(base + off);
    off += round256((size_t)elems * sizeof(float));
  };
  PrefillWorkspace dummy;
  PrefillWorkspace* w = ws ? ws : &dummy;
  take(N * T * HK * S, &w->q);
  take(N * T * HK * S, &w->k);
  take(N * T * H * S, &w->v);
  take(N * T * H, &w->g);
  take(N * T * H, &w->beta);
  take(N * T * H * S, &w->y);
  w->chunk_bytes = gdn_chunked_workspace_bytes((int)N, (int)T, (int)H, (int)S);
  if (base) w->chunk = base + off;
  off += round256(w->chunk_bytes);
  return off;
}

__device__ __forceinline__ void load_bf16x4(const uint16_t* p, float (&x)[4]) {
  const uint2 b = *reinterpret_cast<const uint2*>(p);
  x[0] = bf16_to_float((uint16_t)(b.x & 0xFFFFu));
  x[1] = bf16_to_float((uint16_t)(b.x >> 16));
  x[2] = bf16_to_float((uint16_t)(b.y & 0xFFFFu));
  x[3] = bf16_to_float((uint16_t)(b.y >> 16));
}

template <int K>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_frontend_kernel(
    const uint16_t* __restrict__ qkv, const float* __restrict__ a, const float* __restrict__ b,
    const float* __restrict__ conv_w, const float* __restrict__ ssm_a,
    const float* __restrict__ dt_bias, float* __restrict__ conv_state, float* __restrict__ qo,
    float* __restrict__ ko, float* __restrict__ vo, float* __restrict__ go,
    float* __restrict__ bo, int n_tokens, int n_k_heads, int n_v_heads, int t_chunks,
    int part_blocks, float l2_eps) {
  constexpr int S = kPrefillS, TH = kPrefillTH, TB = kPrefillTB;
  const int lane = threadIdx.x & 63;
  // the wave index is the same in every lane: held in a scalar register, it
  // makes the head part, its kind and every address offset below that does
  // not depend on the lane scalar as well
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, li = lane & 31;
  const int n_parts = 2 * n_k_heads + n_v_heads;
  const int pblk = blockIdx.x % part_blocks;
  const int chunk = (blockIdx.x / part_blocks) % t_chunks;
  const int64_t n = blockIdx.x / ((int64_t)part_blocks * t_chunks);
  const int part = pblk * kPrefillWaves + wv;
  if (part >= n_parts) return;  // a whole wave; the kernel has no barrier

  const int key_dim = n_k_heads * S;
  const int64_t C = 2 * (int64_t)key_dim + (int64_t)n_v_heads * S;
  int kind, head;  // kind 0: q, 1: k, 2: v
  int64_t c0;
  if (part < n_k_heads) {
    kind = 0, head = part, c0 = (int64_t)head * S;
  } else if (part < 2 * n_k_heads) {
    kind = 1, head = part - n_k_heads, c0 = key_dim + (int64_t)head * S;
  } else {
    kind = 2, head = part - 2 * n_k_heads, c0 = 2 * (int64_t)key_dim + (int64_t)head * S;
  }
  const int64_t c = c0 + 4 * li;  // the lane's four channels c .. c+3
  const int t0 = chunk * TB;
  const int tb = t0 + half * TH;  // first position of this half-wave
  const uint16_t* xn = qkv + n * (int64_t)n_tokens * C;
  float* cs = conv_state + (n * C + c) * (K - 1);  // four consecutive histories

  float wc[4][K];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int u = 0; u < K; ++u) wc[j][u] = conv_w[(c + j) * K + u];

  // inputs at positions tb-K+1 .. tb-1 (negative positions: the old history)
  float hist[4][K - 1];
#pragma unroll
  for (int u = 0; u < K - 1; ++u) {
    const int t = tb - (K - 1) + u;
    float xv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (t < 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = cs[j * (K - 1) + (K - 1) + t];
    } else if (t < n_tokens) {
      load_bf16x4(xn + (int64_t)t * C + c, xv);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[j][u] = xv[j];
  }
  const bool owner = (chunk == 0 && half == 0);
  float fin[4][K - 1];
  if (owner) {
#pragma unroll
    for (int u = 0; u < K - 1; ++u) {
      const int t = n_tokens - (K - 1) + u;
      float xv[4];
      if (t < 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = cs[j * (K - 1) + (K - 1) + t];
      } else {
        load_bf16x4(xn + (int64_t)t * C + c, xv);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) fin[j][u] = xv[j];
    }
  }

  // every input of the half-wave's positions, loaded before any arithmetic
  // (positions past the end read the last one and are zeroed at use)
  uint2 xbits[TH];
  const uint16_t* xrow = xn + (int64_t)tb * C + c;
  const uint16_t* xlast = xn + (int64_t)(n_tokens - 1) * C + c;
#pragma unroll
  for (int s = 0; s < TH; ++s) {
    const uint16_t* p = tb + s < n_tokens ? xrow + (int64_t)s * C : xlast;
    xbits[s] = *reinterpret_cast<const uint2*>(p);
  }
  // the decay gate and beta inputs of the wave's positions (v parts)
  const bool gate_lane = (kind == 2 && lane < TB && t0 + lane < n_tokens);
  const int64_t gidx = (n * (int64_t)n_tokens + (gate_lane ? t0 + lane : 0)) * n_v_heads + head;
  float ga = 0.0f, gb = 0.0f, gdt = 0.0f, gsa = 0.0f;
  if (gate_lane) {
    ga = a[gidx];
    gb = b[gidx];
    gdt = dt_bias[head];
    gsa = ssm_a[head];
  }

  // this lane's output row at its half-wave's first position; one position
  // further is one row of the q/k (HK*S) or v (H*S) output further
  const int64_t ostride = kind < 2 ? (int64_t)n_k_heads * S : (int64_t)n_v_heads * S;
  float* obase = (kind == 0 ? qo : kind == 1 ? ko : vo) + (int64_t)head * S +
                 (n * (int64_t)n_tokens + t0) * ostride;
  float* orow = obase + (int64_t)(half * TH) * ostride + 4 * li;
#pragma unroll
  for (int s = 0; s < TH; ++s) {  // the same trip count in every lane: reductions stay whole
    const int t = tb + s;
    const bool valid = t < n_tokens;
    float xv[4];
    xv[0] = bf16_to_float((uint16_t)(xbits[s].x & 0xFFFFu));
    xv[1] = bf16_to_float((uint16_t)(xbits[s].x >> 16));
    xv[2] = bf16_to_float((uint16_t)(xbits[s].y & 0xFFFFu));
    xv[3] = bf16_to_float((uint16_t)(xbits[s].y >> 16));
    if (!valid) xv[0] = xv[1] = xv[2] = xv[3] = 0.0f;
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = conv_point<K>(xv[j], hist[j], wc[j]);
#pragma unroll
      for (int u = 0; u + 1 < K - 1; ++u) hist[j][u] = hist[j][u + 1];
      hist[j][K - 2] = xv[j];
    }
    float* dst = orow + (int64_t)s * ostride;
    if (kind < 2) {
#pragma clang fp contract(off)
      float ss = 0.0f;
      ss = __builtin_fmaf(o[0], o[0], ss);
      ss = __builtin_fmaf(o[1], o[1], ss);
      ss = __builtin_fmaf(o[2], o[2], ss);
      ss = __builtin_fmaf(o[3], o[3], ss);
      ss = group_sum<32>(ss);
      const float inv = inv_l2norm(ss, l2_eps);
      if (valid) store4(dst, make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv));
    } else if (valid) {
      store4(dst, make_float4(o[0], o[1], o[2], o[3]));
    }
  }
  if (owner) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < K - 1; ++u) cs[j * (K - 1) + u] = fin[j][u];
  }
  // decay gate and beta of the wave's positions, by the v parts
  if (gate_lane) {
    go[gidx] = decay_gate(ga, gdt, gsa);
    bo[gidx] = sigmoid(gb);
  }
}

inline int64_t frontend_blocks(int64_t n_seqs, int64_t n_tokens, int64_t n_k_heads,
                               int64_t n_v_heads) {
  return n_seqs * ((n_tokens + kPrefillTB - 1) / kPrefillTB) *
         ((2 * n_k_heads + n_v_heads + kPrefillWaves - 1) / kPrefillWaves);
}

template <int K>
static int launch_frontend(const uint16_t* qkv, const float* a, const float* b,
                           const float* conv_w, const float* ssm_a, const float* dt_bias,
                           float* conv_state, const PrefillWorkspace& ws, int n_seqs, int n_tokens,
                           int n_k_heads, int n_v_heads, float l2_eps, hipStream_t s) {
  const int t_chunks = (n_tokens + kPrefillTB - 1) / kPrefillTB;
  const int part_blocks = (2 * n_k_heads + n_v_heads + kPrefillWaves - 1) / kPrefillWaves;
  const int64_t blocks = frontend_blocks(n_seqs, n_tokens, n_k_heads, n_v_heads);
  return launch(prefill_frontend_kernel<K>, dim3((unsigned)blocks), dim3(64 * kPrefillWaves),
                0, s, qkv, a, b, conv_w, ssm_a, dt_bias, conv_state, ws.q, ws.k, ws.v, ws.g,
                ws.beta, n_tokens, n_k_heads, n_v_heads, t_chunks, part_blocks, l2_eps);
}

}  // namespace gdn

using namespace gdn;

extern "C" size_t gdn_prefill_workspace_bytes(int n_seqs, int n_tokens, int n_k_heads,
                                              int n_v_heads, int state_size) {
  if (n_seqs < 0 || n_tokens < 0 || n_k_heads <= 0 || n_v_heads <= 0 || state_size <= 0) return 0;
  return prefill_layout(n_seqs, n_tokens, n_k_heads, n_v_heads, state_size, nullptr, nullptr);
}

extern "C" int gdn_prefill_bf16_ex(const uint16_t* qkv, const uint16_t* z, const float* a,
                                   const float* b, const float* conv_w, const float* ssm_a,
                                   const float* dt_bias, const float* norm_w, float* conv_state,
                                   float* state, float* out, void* workspace,
                                   size_t workspace_bytes, int n_seqs, int n_tokens,
                                   int n_k_heads, int n_v_heads, int state_size, int conv_kernel,
                                   float scale, float l2_eps, float eps, int scan, void* stream) {
  if (scan != GDN_SCAN_SEQUENTIAL && scan != GDN_SCAN_CHUNKED) return GDN_EUNSUPPORTED;
  if (n_seqs < 0 || n_tokens < 0 || n_k_heads <= 0 || n_v_heads <= 0 || state_size <= 0 ||
      conv_kernel <= 0)
    return GDN_ESIZE;
  if (n_v_heads % n_k_heads != 0) return GDN_ESIZE;
  if (state_size != kPrefillS || conv_kernel < 2 || conv_kernel > 4) return GDN_EUNSUPPORTED;
  if (n_seqs == 0 || n_tokens == 0) return GDN_OK;
  if (!qkv || !z || !a || !b || !conv_w || !ssm_a || !dt_bias || !norm_w || !conv_state ||
      !state || !out || !workspace)
    return GDN_ENULL;
  int64_t rows, elems;
  if (!mul_ok((int64_t)n_seqs * n_tokens, n_v_heads, &rows) || !mul_ok(rows, state_size, &elems))
    return GDN_ESIZE;
  const size_t need = prefill_layout(n_seqs, n_tokens, n_k_heads, n_v_heads, state_size, nullptr,
                                     nullptr);
  if (workspace_bytes < need) return GDN_ESIZE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN_EALIGN;
  if (!aligned16(state) || !aligned16(norm_w) || !aligned16(out)) return GDN_EALIGN;
  if ((reinterpret_cast<uintptr_t>(z) & 7u) != 0 || (reinterpret_cast<uintptr_t>(qkv) & 7u) != 0)
    return GDN_EALIGN;
  // the scan's and the norm's own limits, checked here so that a call they
  // would refuse launches nothing (the front end rolls conv_state in place)
  if (recurrence_size_check(n_seqs, n_tokens, n_v_heads, state_size) != GDN_OK) return GDN_ESIZE;
  if (scan == GDN_SCAN_CHUNKED && chunked_size_check(n_seqs, n_tokens, n_v_heads) != GDN_OK)
    return GDN_ESIZE;
  if (frontend_blocks(n_seqs, n_tokens, n_k_heads, n_v_heads) >= (int64_t(1) << 31))
    return GDN_ESIZE;
  PrefillWorkspace ws;
  prefill_layout(n_seqs, n_tokens, n_k_heads, n_v_heads, state_size,
                 reinterpret_cast<char*>(workspace), &ws);
  hipStream_t s = as_stream(stream);
  int rc = GDN_EUNSUPPORTED;
  switch (conv_kernel) {
    case 2: rc = launch_frontend<2>(qkv, a, b, conv_w, ssm_a, dt_bias, conv_state, ws, n_seqs, n_tokens, n_k_heads, n_v_heads, l2_eps, s); break;
    case 3: rc = launch_frontend<3>(qkv, a, b, conv_w, ssm_a, dt_bias, conv_state, ws, n_seqs, n_tokens, n_k_heads, n_v_heads, l2_eps, s); break;
    case 4: rc = launch_frontend<4>(qkv, a, b, conv_w, ssm_a, dt_bias, conv_state, ws, n_seqs, n_tokens, n_k_heads, n_v_heads, l2_eps, s); break;
  }
  if (rc != GDN_OK) return rc;
  if (scan == GDN_SCAN_CHUNKED)
    rc = gdn_recurrence_seq_chunked(state, ws.q, ws.k, ws.v, ws.g, ws.beta, ws.y, ws.chunk,
                                    ws.chunk_bytes, n_seqs, n_tokens, n_k_heads, n_v_heads,
                                    state_size, scale, stream);
  else
    rc = gdn_recurrence_seq_ex(state, ws.q, ws.k, ws.v, ws.g, ws.beta, ws.y, nullptr, n_seqs,
                               n_tokens, n_k_heads, n_v_heads, state_size, scale,
                               GDN_RECUR_EXACT, stream);
  if (rc != GDN_OK) return rc;
  return launch_gated_rmsnorm_bf16z(ws.y, norm_w, z, out, rows, state_size, eps, s);
}

extern "C" int gdn_prefill_bf16(const uint16_t* qkv, const uint16_t* z, const float* a,
                                const float* b, const float* conv_w, const float* ssm_a,
                                const float* dt_bias, const float* norm_w, float* conv_state,
                                float* state, float* out, void* workspace, size_t workspace_bytes,
                                int n_seqs, int n_tokens, int n_k_heads, int n_v_heads,
                                int state_size, int conv_kernel, float scale, float l2_eps,
                                float eps, void* stream) {
  return gdn_prefill_bf16_ex(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out,
                             workspace, workspace_bytes, n_seqs, n_tokens, n_k_heads, n_v_heads,
                             state_size, conv_kernel, scale, l2_eps, eps, GDN_SCAN_SEQUENTIAL,
                             stream);
}
