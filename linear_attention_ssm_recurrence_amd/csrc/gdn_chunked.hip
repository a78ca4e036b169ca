// Chunked form of the gated delta-rule scan on gfx950, with fp32 MFMA.
//
// The pages name a chunked prefill path and keep the sequential scan as its
// correctness reference (fm_kernel_ssm.m, "softplus" comment and the
// sequential-scan section); they do not give the algorithm. This is the
// standard WY-style blocking of the delta rule, derived from the per-token
// rule itself. For one head and a chunk of C positions with state M0 at the
// chunk start (M is Dv x Dk, row j the stored row j), cumulative log-decay
// Gc_t = sum_{s<=t} g_s, gamma_t = exp(Gc_t):
//   u_t = beta_t (v_t - gamma_t M0 k_t - sum_{s<t} (gamma_t/gamma_s)(k_s.k_t) u_s)
// so with A[t][s] = beta_t (gamma_t/gamma_s)(k_t.k_s) (s < t) and
// X = (I + A)^-1 (unit lower triangular):
//   U  = Tt V - W M0^T,     Tt = X diag(beta),  W = X diag(beta gamma) K
//   Y  = scale (diag(gamma) Q M0^T + P U),  P[t][s] = (gamma_t/gamma_s)(q_t.k_s), s <= t
//   M  = gamma_C M0 + U^T Kt,  Kt[s] = (gamma_C/gamma_s) k_s
// (U, V, Y are C x Dv with rows per position; Q, K are C x Dk.)
//
// Two kernels:
//  chunk_prep_kernel  one block per (sequence, V-head, chunk), all chunks in
//                     parallel: Gc, then K K^T and Q K^T (lower tiles, MFMA),
//                     A and P, X by forward substitution (4 lanes per column),
//                     W (MFMA). Writes Gc, Tt, P, W to the workspace.
//  chunk_scan_kernel  one block per (sequence, V-head, 16 state rows), the
//                     chunks in order: the 16 rows stay on chip, and per chunk
//                     each of the 4 waves does 128 MFMAs (U, Y, state update).
// Positions past the end of the sequence in the last chunk are padded with
// g = 0, beta = 0 and k = q = 0: their rows of A, W and U are zero, so they
// leave the state unchanged, and their y are not stored.
//
// MFMA v_mfma_f32_16x16x4f32 (checked on MI355X): lane l supplies
// A[l%16][l/16] and B[l/16][l%16]; output element i of lane l is
// D[4*(l/16) + i][l%16]. A dot product's k range is split as
// k = (l/16)*KS + kk over the MFMA steps kk (KS = K/4), which makes the
// operands of consecutive steps contiguous in memory: each lane reads them as
// float4. Accumulation order therefore differs from the sequential scan;
// results agree with it within the fp32 tolerance, not bit for bit.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kChS = 128;     // state size
constexpr int kChC = 64;      // chunk length
constexpr int kChR = 16;      // state rows per scan block
constexpr int kChUnit = kChC + 2 * kChC * kChC + kChC * kChS;  // floats per (seq, head, chunk)

__device__ __forceinline__ f32x4v mfma4(float a, float b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct ChunkUnit {   // views into one unit of the workspace
  float* gc;  // [C]
  float* tt;  // [C][C]   X diag(beta)
  float* p;   // [C][C]   (gamma_t/gamma_s) q_t.k_s, s <= t
  float* w;   // [C][S]   X diag(beta gamma) K
};

__device__ __forceinline__ ChunkUnit chunk_unit(float* ws, int64_t unit) {
  float* base = ws + unit * kChUnit;
  return {base, base + kChC, base + kChC + kChC * kChC, base + kChC + 2 * kChC * kChC};
}

// ---------------------------------------------------------------------------
// Chunk preparation
// ---------------------------------------------------------------------------
constexpr int kKP = kChS + 4;   // LDS row pitch of K and Q (floats)
constexpr int kAP = kChC + 4;   // LDS row pitch of A and X

__global__ __launch_bounds__(256) void chunk_prep_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, float* __restrict__ ws, int n_tokens, int n_k_heads,
    int n_v_heads, int n_chunks) {
  constexpr int S = kChS, C = kChC;
  constexpr int QS = (C * kKP > 2 * C * kAP) ? C * kKP : 2 * C * kAP;
  __shared__ float Ks[C * kKP];
  __shared__ float Qs[QS];        // reused for A and X once Q K^T is done
  __shared__ float Gs[C], Bs[C], BG[C];
  float* As = Qs;                 // [C][kAP]
  float* Xs = Qs + C * kAP;       // [C][kAP]

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t unit = blockIdx.x;                    // (n * H + h) * n_chunks + c
  const int chunk = (int)(unit % n_chunks);
  const int64_t head = unit / n_chunks;               // n * H + h
  const int64_t n = head / n_v_heads;
  const int h = (int)(head % n_v_heads);
  const int kh = h % n_k_heads;
  const int t0 = chunk * C;
  const int64_t kq_tok = (int64_t)n_k_heads * S;
  const float* kn = k + (n * n_tokens) * kq_tok + (int64_t)kh * S;
  const float* qn = q + (n * n_tokens) * kq_tok + (int64_t)kh * S;
  ChunkUnit u = chunk_unit(ws, unit);

  // K and Q of the chunk (zero past the end)
  for (int f = tid * 4; f < C * S; f += 256 * 4) {
    const int t = f / S, col = f % S;
    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
    if (t0 + t < n_tokens) {
      kv = load4(kn + (int64_t)(t0 + t) * kq_tok + col);
      qv = load4(qn + (int64_t)(t0 + t) * kq_tok + col);
    }
    store4(Ks + t * kKP + col, kv);
    store4(Qs + t * kKP + col, qv);
  }
  // cumulative log-decay and beta (wave 0; sequential prefix sum by lane 0)
  if (wv == 0) {
    const int t = t0 + lane;
    const bool ok = t < n_tokens;
    const int64_t gi = (n * n_tokens + t) * n_v_heads + h;
    Gs[lane] = ok ? g[gi] : 0.0f;
    Bs[lane] = ok ? beta[gi] : 0.0f;
  }
  __syncthreads();
  if (tid == 0) {
    float acc = 0.0f;
    for (int t = 0; t < C; ++t) {
      acc += Gs[t];
      Gs[t] = acc;
    }
  }
  __syncthreads();
  if (tid < C) {
    u.gc[tid] = Gs[tid];
    BG[tid] = Bs[tid] * expf(Gs[tid]);   // beta_s gamma_s
  }

  // K K^T and Q K^T on the lower tiles (ti >= tj): 10 tiles each, 20 per
  // block, 5 per wave (tile id = wv + 4m: ids 0..9 are K K^T, 10..19 Q K^T)
  const int g4 = lane >> 4, l16 = lane & 15;
  auto tile_of = [](int idx, int& ti, int& tj) {
    const int tix = idx % 10;
    ti = 0, tj = tix;
    while (tj > ti) {
      tj -= ti + 1;
      ++ti;
    }
  };
  f32x4v acc5[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int idx = wv + 4 * m;
    int ti, tj;
    tile_of(idx, ti, tj);
    const float* Arow = (idx < 10 ? Ks : Qs) + (ti * 16 + l16) * kKP + g4 * (S / 4);
    const float* Brow = Ks + (tj * 16 + l16) * kKP + g4 * (S / 4);
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < S / 4; kk += 4) {
      const float4 a4 = load4(Arow + kk);
      const float4 b4 = load4(Brow + kk);
      acc = mfma4(a4.x, b4.x, acc);
      acc = mfma4(a4.y, b4.y, acc);
      acc = mfma4(a4.z, b4.z, acc);
      acc = mfma4(a4.w, b4.w, acc);
    }
    acc5[m] = acc;
  }
  __syncthreads();   // Q no longer needed: As and Xs overwrite Qs
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int idx = wv + 4 * m;
    int ti, tj;
    tile_of(idx, ti, tj);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = ti * 16 + g4 * 4 + i, s = tj * 16 + l16;
      const float r = expf(Gs[t] - Gs[s]);
      if (idx < 10) {
        As[t * kAP + s] = (s < t) ? Bs[t] * r * acc5[m][i] : 0.0f;
      } else {
        u.p[t * C + s] = (s <= t) ? r * acc5[m][i] : 0.0f;
      }
    }
  }
  // upper tiles: A is not read there; P is stored as zero
  for (int f = tid; f < C * C; f += 256) {
    const int t = f / C, s = f % C;
    if ((s >> 4) > (t >> 4)) u.p[f] = 0.0f;
  }
  __syncthreads();

  // X = (I + A)^-1, column by column; four lanes per column split the sum
  {
    const int col = tid >> 2, part = tid & 3;
    for (int t = 0; t < C; ++t) {
      float acc = 0.0f;
      for (int s = part; s < t; s += 4) acc = __builtin_fmaf(As[t * kAP + s], Xs[s * kAP + col], acc);
      acc = acc + dpp_mov<kDppQuadXor1>(acc);
      acc = acc + dpp_mov<kDppQuadXor2>(acc);
      if (part == 0) Xs[t * kAP + col] = (t == col ? 1.0f : 0.0f) - acc;
      __syncthreads();
    }
  }
  // Tt = X diag(beta)
  for (int f = tid; f < C * C; f += 256) {
    const int t = f / C, s = f % C;
    u.tt[f] = Xs[t * kAP + s] * Bs[s];
  }
  // W = X diag(beta gamma) K: 4 x 8 output tiles of 16 x 16, 8 per wave
  for (int tile = wv; tile < 32; tile += 4) {
    const int ti = tile >> 3, tc = tile & 7;
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C / 4; ++kk) {
      const int s = g4 * (C / 4) + kk;
      const float a = Xs[(ti * 16 + l16) * kAP + s] * BG[s];
      const float b = Ks[s * kKP + tc * 16 + l16];
      acc = mfma4(a, b, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) u.w[(ti * 16 + g4 * 4 + i) * S + tc * 16 + l16] = acc[i];
  }
}

// ---------------------------------------------------------------------------
// Chunk scan
// ---------------------------------------------------------------------------
constexpr int kMP = kChS + 4;   // LDS pitch of the state rows
constexpr int kUP = kChR + 4;   // LDS pitch of U and V

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void chunk_scan_kernel(float* __restrict__ state, const float* __restrict__ q,
                       const float* __restrict__ k, const float* __restrict__ v,
                       const float* __restrict__ ws, float* __restrict__ y, int n_tokens,
                       int n_k_heads, int n_v_heads, int n_chunks, float scale) {
  constexpr int S = kChS, C = kChC, R = kChR;
  __shared__ float Ms[R * kMP];
  __shared__ float Us[C * kUP];
  __shared__ float Vs[C * kUP];
  __shared__ float Gam[C];   // gamma_t = exp(Gc_t)
  __shared__ float Ktf[C];   // gamma_C / gamma_s = exp(Gc_C - Gc_s)

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int64_t head = blockIdx.x / (S / R);          // n * H + h
  const int row0 = (int)(blockIdx.x % (S / R)) * R;
  const int64_t n = head / n_v_heads;
  const int h = (int)(head % n_v_heads);
  const int kh = h % n_k_heads;
  const int64_t kq_tok = (int64_t)n_k_heads * S, v_tok = (int64_t)n_v_heads * S;
  const float* kn = k + (n * n_tokens) * kq_tok + (int64_t)kh * S;
  const float* qn = q + (n * n_tokens) * kq_tok + (int64_t)kh * S;
  const float* vn = v + (n * n_tokens) * v_tok + (int64_t)h * S + row0;
  float* yn = y + (n * n_tokens) * v_tok + (int64_t)h * S + row0;
  float* sp = state + head * (int64_t)S * S + (int64_t)row0 * S;

  // state rows: LDS copy (B operand of M^T products) and this wave's two
  // 16 x 16 column tiles in the MFMA output layout (the update accumulators)
  for (int f = tid * 4; f < R * S; f += 256 * 4) store4(Ms + (f / S) * kMP + f % S, load4(sp + f));
  f32x4v macc[2];
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int i = 0; i < 4; ++i) macc[c2][i] = sp[(g4 * 4 + i) * S + (wv * 2 + c2) * 16 + l16];

  for (int chunk = 0; chunk < n_chunks; ++chunk) {
    const int t0 = chunk * C;
    const ChunkUnit u = chunk_unit(const_cast<float*>(ws), head * n_chunks + chunk);
    // V of the block's rows (zero past the end), and Gc
    {
      const int t = tid >> 2, c4 = (tid & 3) * 4;
      float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t0 + t < n_tokens) vv = load4(vn + (int64_t)(t0 + t) * v_tok + c4);
      store4(Vs + t * kUP + c4, vv);
      if (tid < C) {
        const float gc = u.gc[tid];
        Gam[tid] = expf(gc);
        Ktf[tid] = expf(u.gc[C - 1] - gc);
      }
    }
    __syncthreads();

    // U rows 16wv..16wv+15 = Tt V - W M^T ; Y part = gamma Q M^T
    const int trow = wv * 16 + l16;                   // this lane's A-operand row
    const bool tok_ok = t0 + trow < n_tokens;
    f32x4v uacc = {0.f, 0.f, 0.f, 0.f}, yacc = {0.f, 0.f, 0.f, 0.f};
    {
      const float* ttr = u.tt + trow * C + g4 * (C / 4);
#pragma unroll
      for (int kk = 0; kk < C / 4; kk += 4) {
        const float4 a4 = load4(ttr + kk);
        const int s = g4 * (C / 4) + kk;
        uacc = mfma4(a4.x, Vs[(s + 0) * kUP + l16], uacc);
        uacc = mfma4(a4.y, Vs[(s + 1) * kUP + l16], uacc);
        uacc = mfma4(a4.z, Vs[(s + 2) * kUP + l16], uacc);
        uacc = mfma4(a4.w, Vs[(s + 3) * kUP + l16], uacc);
      }
      const float* wr = u.w + trow * S + g4 * (S / 4);
      const float* qr = qn + (int64_t)(t0 + trow) * kq_tok + g4 * (S / 4);
      const float* mr = Ms + l16 * kMP + g4 * (S / 4);
      const float gam = Gam[trow];
#pragma unroll
      for (int kk = 0; kk < S / 4; kk += 4) {
        const float4 w4 = load4(wr + kk);
        const float4 m4 = load4(mr + kk);
        float4 q4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tok_ok) q4 = load4(qr + kk);
        uacc = mfma4(-w4.x, m4.x, uacc);
        yacc = mfma4(gam * q4.x, m4.x, yacc);
        uacc = mfma4(-w4.y, m4.y, uacc);
        yacc = mfma4(gam * q4.y, m4.y, yacc);
        uacc = mfma4(-w4.z, m4.z, uacc);
        yacc = mfma4(gam * q4.z, m4.z, yacc);
        uacc = mfma4(-w4.w, m4.w, uacc);
        yacc = mfma4(gam * q4.w, m4.w, yacc);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Us[(wv * 16 + g4 * 4 + i) * kUP + l16] = uacc[i];
    __syncthreads();

    // Y += P U ; y out
    {
      const float* pr = u.p + trow * C + g4 * (C / 4);
#pragma unroll
      for (int kk = 0; kk < C / 4; kk += 4) {
        const float4 a4 = load4(pr + kk);
        const int s = g4 * (C / 4) + kk;
        yacc = mfma4(a4.x, Us[(s + 0) * kUP + l16], yacc);
        yacc = mfma4(a4.y, Us[(s + 1) * kUP + l16], yacc);
        yacc = mfma4(a4.z, Us[(s + 2) * kUP + l16], yacc);
        yacc = mfma4(a4.w, Us[(s + 3) * kUP + l16], yacc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + wv * 16 + g4 * 4 + i;
        if (t < n_tokens) yn[(int64_t)t * v_tok + l16] = scale * yacc[i];
      }
    }
    // state update of this wave's column tiles: M = gamma_C M + U^T Kt
    {
      const float gam_c = Gam[C - 1];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int col = (wv * 2 + c2) * 16 + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) macc[c2][i] *= gam_c;
#pragma unroll
        for (int kk = 0; kk < C / 4; ++kk) {
          const int s = g4 * (C / 4) + kk;
          const float a = Us[s * kUP + l16];
          float b = 0.0f;
          if (t0 + s < n_tokens) b = kn[(int64_t)(t0 + s) * kq_tok + col] * Ktf[s];
          macc[c2] = mfma4(a, b, macc[c2]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Ms[(g4 * 4 + i) * kMP + col] = macc[c2][i];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int i = 0; i < 4; ++i) sp[(g4 * 4 + i) * S + (wv * 2 + c2) * 16 + l16] = macc[c2][i];
}

}  // namespace gdn

using namespace gdn;

extern "C" size_t gdn_chunked_workspace_bytes(int n_seqs, int n_tokens, int n_v_heads,
                                              int state_size) {
  if (n_seqs < 0 || n_tokens < 0 || n_v_heads <= 0 || state_size != kChS) return 0;
  const int64_t chunks = (n_tokens + kChC - 1) / kChC;
  return (size_t)n_seqs * n_v_heads * chunks * kChUnit * sizeof(float);
}

extern "C" int gdn_recurrence_seq_chunked(float* state, const float* q, const float* k,
                                          const float* v, const float* g, const float* beta,
                                          float* y, void* workspace, size_t workspace_bytes,
                                          int n_seqs, int n_tokens, int n_k_heads, int n_v_heads,
                                          int state_size, float scale, void* stream) {
  if (n_seqs < 0 || n_tokens < 0 || n_k_heads <= 0 || n_v_heads <= 0 || state_size <= 0)
    return GDN_ESIZE;
  if (n_v_heads % n_k_heads != 0) return GDN_ESIZE;
  if (state_size != kChS) return GDN_EUNSUPPORTED;
  if (n_seqs == 0 || n_tokens == 0) return GDN_OK;
  if (!state || !q || !k || !v || !g || !beta || !y || !workspace) return GDN_ENULL;
  const size_t need = gdn_chunked_workspace_bytes(n_seqs, n_tokens, n_v_heads, state_size);
  if (workspace_bytes < need) return GDN_ESIZE;
  if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(workspace))
    return GDN_EALIGN;
  const int n_chunks = (n_tokens + kChC - 1) / kChC;
  const int64_t units = (int64_t)n_seqs * n_v_heads * n_chunks;
  const int64_t scan_blocks = (int64_t)n_seqs * n_v_heads * (kChS / kChR);
  if (units >= (int64_t(1) << 31) || scan_blocks >= (int64_t(1) << 31)) return GDN_ESIZE;
  hipStream_t s = as_stream(stream);
  float* ws = reinterpret_cast<float*>(workspace);
  hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)units), dim3(256), 0, s, q, k, g, beta, ws,
                     n_tokens, n_k_heads, n_v_heads, n_chunks);
  int rc = launch_status();
  if (rc != GDN_OK) return rc;
  hipLaunchKernelGGL(chunk_scan_kernel, dim3((unsigned)scan_blocks), dim3(256), 0, s, state, q, k,
                     v, ws, y, n_tokens, n_k_heads, n_v_heads, n_chunks, scale);
  return launch_status();
}
