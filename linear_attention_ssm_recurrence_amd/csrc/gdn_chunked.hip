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
//   U  = X Z,   Z = diag(beta) V - diag(beta gamma) K M0^T
//   Y  = scale (diag(gamma) Q M0^T + P U),  P[t][s] = (gamma_t/gamma_s)(q_t.k_s), s <= t
//   M  = gamma_C M0 + (diag(gamma_C/gamma) U)^T K
// (U, V, Y are C x Dv with rows per position; Q, K are C x Dk.)
//
// Two kernels:
//  chunk_prep_kernel  one block per (sequence, K-head, chunk), all chunks in
//                     parallel: K K^T and Q K^T (lower tiles, MFMA) once per
//                     K-head, then for each V-head that reads it: Gc (summed
//                     in fp64: under strong decay it reaches thousands, where
//                     an fp32 difference Gc_t - Gc_s would lose ~1e-4), A and
//                     P, X blockwise (16 x 16 diagonal tiles by forward
//                     substitution, the others by MFMA). Writes gamma,
//                     gamma_C/gamma, beta, X and P of every V-head to the
//                     workspace. Q is read as register fragments and K's LDS
//                     region is reused for A and X, so a block needs ~39 KB
//                     (four per CU).
//  chunk_scan_kernel  one block per (sequence, V-head, 16 state rows), the
//                     chunks in order: the 16 rows stay on chip, and per chunk
//                     each of the 4 waves does 128 MFMAs (K M^T and Q M^T,
//                     X Z, P U, the state update).
// Positions past the end of the sequence in the last chunk are padded with
// g = 0 and beta = 0 in the preparation, and their q and k rows repeat the
// last valid position: their rows of A, Z and U, and their entries of beta,
// are zero, so they leave the state unchanged, and a valid row t meets them
// neither in A nor in P (both take s <= t). Their rows of P and y are not
// used: those y are not stored.
//
// MFMA v_mfma_f32_16x16x4f32 (checked on MI355X): lane l supplies
// A[l%16][l/16] and B[l/16][l%16]; output element i of lane l is
// D[4*(l/16) + i][l%16]. The scan splits a dot product's k range as
// k = 16j + 4*(l/16) + c over the MFMA steps (j, c): a lane's operands for
// four consecutive steps are contiguous (one float4), the four lane groups of
// a row read 64 contiguous bytes, and LDS reads of a pitch-4 (mod 8) array
// see only the unavoidable 2-way bank split. The workspace matrices are
// stored in that lane order ("fragment order": 16 x 16 tiles of 256 floats,
// float4 of lane l at 4l), so each operand load is one contiguous 1 KB.
// Accumulation order differs from the sequential scan; results agree with it
// within the fp32 tolerance, not bit for bit.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kChS = 128;     // state size
constexpr int kChC = 64;      // chunk length
constexpr int kChR = 16;      // state rows per scan block
constexpr int kChHead = 4 * kChC;                                   // per-position factors
constexpr int kChUnit = kChHead + 2 * kChC * kChC;                  // floats per (seq, head, chunk)

__device__ __forceinline__ f32x4v mfma4(float a, float b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct ChunkUnit {   // views into one unit of the workspace
  float* gam; // [C]      gamma_t = exp(Gc_t)
  float* ktf; // [C]      gamma_C / gamma_s
  float* bet; // [C]      beta_t (0 past the end)
  float* x;   // [C][C]   (I + A)^-1, fragment order
  float* p;   // [C][C]   (gamma_t/gamma_s) q_t.k_s for s <= t, else 0; fragment order
};

// Offset of element (r, c) of a 16 x 16 tile in fragment order.
__device__ __forceinline__ int frag_off(int r, int c) {
  return (((c >> 2) & 3) * 16 + r) * 4 + (c & 3);
}
// Offset of element (t, s) of a matrix with nj 16-column tiles per tile row.
__device__ __forceinline__ int frag_index(int t, int s, int nj) {
  return ((t >> 4) * nj + (s >> 4)) * 256 + frag_off(t & 15, s & 15);
}

__device__ __forceinline__ ChunkUnit chunk_unit(float* ws, int64_t unit) {
  float* base = ws + unit * kChUnit;
  float* mats = base + kChHead;
  return {base, base + kChC, base + 2 * kChC, mats, mats + kChC * kChC};
}

// ---------------------------------------------------------------------------
// Chunk preparation
// ---------------------------------------------------------------------------
constexpr int kKP = kChS + 4;   // LDS row pitch of K (floats)
constexpr int kAP = kChC + 4;   // LDS row pitch of A and X
constexpr int kTP = 16 + 4;     // LDS row pitch of a 16 x 16 scratch tile

__global__ __launch_bounds__(256) void chunk_prep_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, float* __restrict__ ws, int n_tokens, int n_k_heads,
    int n_v_heads, int n_chunks, int v_groups) {
  constexpr int S = kChS, C = kChC;
  constexpr int AXT = 2 * C * kAP + 3 * 16 * kTP;   // A, X and three scratch tiles
  constexpr int SM = (C * kKP > AXT) ? C * kKP : AXT;
  // One LDS region: K during the Gram tiles, then A, X and the scratch tiles.
  // Q never goes through LDS (the Q K^T waves take their rows as register
  // fragments), which keeps a block at ~39 KB: four blocks per CU.
  __shared__ float Sm[SM];
  __shared__ double Gs[C];        // Gc in fp64: differences of large sums keep their precision
  __shared__ float Bs[C];
  float* Ks = Sm;                 // [C][kKP]
  float* As = Sm;                 // [C][kAP]
  float* Xs = Sm + C * kAP;       // [C][kAP]
  float* Ts = Sm + 2 * C * kAP;   // [3][16][kTP]

  // One block per (sequence, K-head, V-head group, chunk). K K^T and Q K^T
  // depend only on the K-head, so they are computed once and kept in
  // registers; A, P and X, which take each V-head's gate and beta, are then
  // formed for the block's V-heads kh + r*HK, r in [r0, r1) (V-head h reads
  // K-head h mod HK), one after the other. The V-heads of a K-head are split
  // over v_groups blocks only when one block per K-head would leave the chip
  // short of blocks.
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t unit = blockIdx.x;                    // ((n * HK + kh) * v_groups + vg) * n_chunks + c
  const int chunk = (int)(unit % n_chunks);
  const int vg = (int)((unit / n_chunks) % v_groups);
  const int64_t khead = unit / n_chunks / v_groups;   // n * HK + kh
  const int64_t n = khead / n_k_heads;
  const int kh = (int)(khead % n_k_heads);
  const int per_group = n_v_heads / n_k_heads / v_groups;
  const int r0 = vg * per_group, r1 = r0 + per_group;
  const int t0 = chunk * C;
  const int64_t kq_tok = (int64_t)n_k_heads * S;
  const float* kn = k + (n * n_tokens) * kq_tok + (int64_t)kh * S;
  const float* qn = q + (n * n_tokens) * kq_tok + (int64_t)kh * S;

  // Gram tiles (lower tiles only, ti >= tj): the Q-waves (0, 1) compute
  // Q K^T, the K-waves (2, 3) K K^T, each on the tiles of two tile rows,
  // {0, 3} (even waves) or {1, 2} (odd waves): five tiles per wave.
  const int g4 = lane >> 4, l16 = lane & 15;
  const bool qwave = wv < 2;
  const int par = wv & 1;
  auto tile_at = [&](int m, int& ti, int& tj) {
    if (par == 0) {
      ti = m == 0 ? 0 : 3;
      tj = m == 0 ? 0 : m - 1;
    } else {
      ti = m < 2 ? 1 : 2;
      tj = m < 2 ? m : m - 2;
    }
  };
  // Q rows of the two tile rows as A fragments (k = 16j + 4*(l/16) + c),
  // loaded first; rows past the end read the last position (their P rows are
  // never used: those y are not stored)
  float4 qa[8], qb[8];
  if (qwave) {
    const int last = n_tokens - 1;
    const int ta = t0 + (par ? 1 : 0) * 16 + l16, tb = t0 + (par ? 2 : 3) * 16 + l16;
    const float* qra = qn + (int64_t)(ta < last ? ta : last) * kq_tok + 4 * g4;
    const float* qrb = qn + (int64_t)(tb < last ? tb : last) * kq_tok + 4 * g4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qa[j] = load4(qra + 16 * j);
      qb[j] = load4(qrb + 16 * j);
    }
  }
  // K of the chunk: all eight float4 loads of a thread are in flight
  // together. Rows past the end repeat the last position; their beta is 0,
  // so their rows of A are zero, and no valid row t reads them (A and P use
  // s <= t).
  constexpr int KF = C * S / (256 * 4);
  float4 kv[KF];
#pragma unroll
  for (int i = 0; i < KF; ++i) {
    const int f = (tid + 256 * i) * 4, t = f / S, col = f % S;
    const int tt = t0 + t < n_tokens ? t0 + t : n_tokens - 1;
    kv[i] = load4(kn + (int64_t)tt * kq_tok + col);
  }
  // g and beta of one V-head over the chunk (wave 0), issued after K:
  // outstanding loads complete in issue order, so K's stores below do not
  // wait for them
  const bool valid = t0 + lane < n_tokens;
  const int64_t g_row = (n * n_tokens + (valid ? t0 + lane : n_tokens - 1)) * n_v_heads;
  float g_raw = 0.0f, b_raw = 0.0f;
  auto load_gate = [&](int h) {
    if (wv == 0) {
      g_raw = g[g_row + h];
      b_raw = beta[g_row + h];
    }
  };
  // cumulative log-decay (inclusive prefix sum across wave 0) and beta
  // g below -1e4, -inf included (the gate's output when exp(A_log)
  // overflows), enters the sum as -1e4: its decay is exactly 0 in fp32 either
  // way, and a finite value keeps every difference Gc_t - Gc_s exact, where an
  // infinite one would make the differences after it -inf - (-inf) = NaN.
  // (The comparison leaves a NaN g NaN.)
  auto prefix = [&]() {
    if (wv == 0) {
      const double gv = g_raw < -1.0e4f ? -1.0e4 : (double)g_raw;
      double gc = valid ? gv : 0.0;
#pragma unroll
      for (int off = 1; off < C; off <<= 1) {
        const double up = __shfl_up(gc, off);
        gc = lane >= off ? gc + up : gc;
      }
      Gs[lane] = gc;
      Bs[lane] = valid ? b_raw : 0.0f;
    }
  };
  load_gate(kh + r0 * n_k_heads);
#pragma unroll
  for (int i = 0; i < KF; ++i) {
    const int f = (tid + 256 * i) * 4, t = f / S, col = f % S;
    store4(Ks + t * kKP + col, kv[i]);
  }
  prefix();
  __syncthreads();

  f32x4v acc5[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    int ti, tj;
    tile_at(m, ti, tj);
    const float* Brow = Ks + (tj * 16 + l16) * kKP + 4 * g4;
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
    if (qwave) {
      const bool first_row = (par == 0) ? (m == 0) : (m < 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 a4 = first_row ? qa[j] : qb[j];
        const float4 b4 = load4(Brow + 16 * j);
        acc = mfma4(a4.x, b4.x, acc);
        acc = mfma4(a4.y, b4.y, acc);
        acc = mfma4(a4.z, b4.z, acc);
        acc = mfma4(a4.w, b4.w, acc);
      }
    } else {
      const float* Arow = Ks + (ti * 16 + l16) * kKP + 4 * g4;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 a4 = load4(Arow + 16 * j);
        const float4 b4 = load4(Brow + 16 * j);
        acc = mfma4(a4.x, b4.x, acc);
        acc = mfma4(a4.y, b4.y, acc);
        acc = mfma4(a4.z, b4.z, acc);
        acc = mfma4(a4.w, b4.w, acc);
      }
    }
    acc5[m] = acc;
  }
  __syncthreads();   // K no longer needed: A and X overwrite it

  for (int r = r0; r < r1; ++r) {
    // The lane indices of the body come from a copy the compiler cannot see
    // through, so its address arithmetic is redone per V-head instead of
    // being hoisted out of the loop, where it would hold some fifty
    // registers through every iteration.
    int tid_r = tid;
    asm volatile("" : "+v"(tid_r));
    const int g4r = (tid_r & 63) >> 4, l16r = tid_r & 15;
    const int h = kh + r * n_k_heads;
    const ChunkUnit u = chunk_unit(ws, ((n * n_v_heads + h) * n_chunks + chunk));
    if (r + 1 < r1) load_gate(h + n_k_heads);   // lands during this V-head's work
    if (tid_r < C) {
      u.gam[tid_r] = expf((float)Gs[tid_r]);
      u.ktf[tid_r] = expf((float)(Gs[C - 1] - Gs[tid_r]));
      u.bet[tid_r] = Bs[tid_r];
    }
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      int ti, tj;
      tile_at(m, ti, tj);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = ti * 16 + g4r * 4 + i, s = tj * 16 + l16r;
        const float rr = expf((float)(Gs[t] - Gs[s]));
        if (qwave) {
          u.p[frag_index(t, s, 4)] = (s <= t) ? rr * acc5[m][i] : 0.0f;
        } else {
          As[t * kAP + s] = (s < t) ? Bs[t] * rr * acc5[m][i] : 0.0f;
        }
      }
    }
    // upper tiles: A is not read there; P is stored as zero (whole tiles)
    for (int f = tid_r; f < 16 * 256; f += 256) {
      const int tile = f >> 8, ti = tile >> 2, tj = tile & 3;
      if (tj > ti) u.p[f] = 0.0f;
    }
    __syncthreads();

    // X = (I + A)^-1 blockwise on 16 x 16 tiles. Diagonal tiles: wave w
    // inverts tile (w, w) by forward substitution, one column per lane (the
    // four 16-lane groups compute the same columns; group 0 stores them).
    {
      const int b = wv, col = l16r;
      float xr[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float* arow = As + (16 * b + t) * kAP + 16 * b;
        float acc = 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < t; ++s2) acc = __builtin_fmaf(arow[s2], xr[s2], acc);
        xr[t] = (t == col ? 1.0f : 0.0f) - acc;
      }
      if (g4r == 0) {
#pragma unroll
        for (int t = 0; t < 16; ++t) Xs[(16 * b + t) * kAP + 16 * b + col] = xr[t];
      }
      for (int f = tid_r; f < C * C; f += 256) {   // X is lower block-triangular
        const int t = f / C, s2 = f % C;
        if ((s2 >> 4) > (t >> 4)) Xs[t * kAP + s2] = 0.0f;
      }
    }
    __syncthreads();
    // Off-diagonal tiles, one block row at a time:
    //   X_ij = -X_ii (sum_{j <= m < i} A_im X_mj),   wave j computes tile (i, j)
    for (int bi = 1; bi < 4; ++bi) {
      const int bj = wv;
      if (bj < bi) {
        f32x4v acc = {0.f, 0.f, 0.f, 0.f};
        for (int bm = bj; bm < bi; ++bm) {
          const float4 a4 = load4(As + (16 * bi + l16r) * kAP + 16 * bm + 4 * g4r);
          const float* xb = Xs + (16 * bm + 4 * g4r) * kAP + 16 * bj + l16r;
          acc = mfma4(a4.x, xb[0 * kAP], acc);
          acc = mfma4(a4.y, xb[1 * kAP], acc);
          acc = mfma4(a4.z, xb[2 * kAP], acc);
          acc = mfma4(a4.w, xb[3 * kAP], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Ts[(bj * 16 + 4 * g4r + i) * kTP + l16r] = acc[i];
      }
      __syncthreads();
      if (bj < bi) {
        const float4 x4 = load4(Xs + (16 * bi + l16r) * kAP + 16 * bi + 4 * g4r);
        const float* tb = Ts + (bj * 16 + 4 * g4r) * kTP + l16r;
        f32x4v acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma4(x4.x, tb[0 * kTP], acc);
        acc = mfma4(x4.y, tb[1 * kTP], acc);
        acc = mfma4(x4.z, tb[2 * kTP], acc);
        acc = mfma4(x4.w, tb[3 * kTP], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) Xs[(16 * bi + 4 * g4r + i) * kAP + 16 * bj + l16r] = -acc[i];
      }
      __syncthreads();
    }
    // X, written in fragment order (one float4 per thread and step)
    for (int f4 = tid_r; f4 < C * C / 4; f4 += 256) {
      const int tile = f4 >> 6, ln = f4 & 63;
      const int t = (tile >> 2) * 16 + (ln & 15), s0 = (tile & 3) * 16 + (ln >> 4) * 4;
      store4(u.x + 4 * f4, load4(Xs + t * kAP + s0));
    }
    // the next V-head's prefix sum; Gs and Bs were last read before the
    // barriers above, and the barrier below orders the X write-out before
    // the next iteration overwrites As and Xs
    if (r + 1 < r1) {
      prefix();
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk scan
// ---------------------------------------------------------------------------
constexpr int kMP = kChS + 4;   // LDS pitch of the state rows
constexpr int kUP = kChR + 4;   // LDS pitch of U and V
constexpr int kKSP = kChS + 4;  // LDS pitch of the chunk's K

// What one chunk needs from memory, per lane: the A-operand fragments of X
// and P (4 float4 each) from the workspace, the lane's q row pieces (8), and
// this thread's share of K (8 float4) and V (1) for LDS staging. Each group
// is refilled with the next chunk's values right after its last use, so the
// loads overlap the rest of the chunk.
struct ChunkRegs {
  float4 x[4], p[4], q[8], kst[8], v;
  float gam, ktf, bet;
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void chunk_scan_kernel(float* __restrict__ state, const float* __restrict__ q,
                       const float* __restrict__ k, const float* __restrict__ v,
                       const float* __restrict__ ws, float* __restrict__ y, int n_tokens,
                       int n_k_heads, int n_v_heads, int n_chunks, float scale) {
  constexpr int S = kChS, C = kChC, R = kChR;
  __shared__ float Ms[R * kMP];
  __shared__ float Zs[C * kUP];   // Z = diag(beta) V - diag(beta gamma) K M^T
  __shared__ float Us[C * kUP];   // U
  __shared__ float Uk[C * kUP];   // diag(gamma_C / gamma) U, for the state update
  __shared__ float Ys[C * kUP];   // y of the chunk, stored after the chunk's last barrier
  // K, V and the factors of the chunk, staged at the top of each chunk. One
  // buffer keeps the block at ~69 KB of LDS, so two blocks share a CU when
  // there are more blocks than CUs (their waves are not tied by barriers);
  // a second buffer (one barrier less per chunk) measured no faster.
  __shared__ float Vs[C * kUP];
  __shared__ float Ks[C * kKSP];
  __shared__ float Gam[C];        // gamma_t
  __shared__ float Ktf[C];        // gamma_C / gamma_s
  __shared__ float Bet[C];        // beta_t

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  // the S/R blocks of one head read the same operands: keep them on one XCD
  const unsigned blk = xcd_group(blockIdx.x, gridDim.x);
  const int64_t head = blk / (S / R);                 // n * H + h
  const int row0 = (int)(blk % (S / R)) * R;
  const int64_t n = head / n_v_heads;
  const int h = (int)(head % n_v_heads);
  const int kh = h % n_k_heads;
  const int64_t kq_tok = (int64_t)n_k_heads * S, v_tok = (int64_t)n_v_heads * S;
  const float* kn = k + (n * n_tokens) * kq_tok + (int64_t)kh * S;
  const float* qn = q + (n * n_tokens) * kq_tok + (int64_t)kh * S;
  const float* vn = v + (n * n_tokens) * v_tok + (int64_t)h * S + row0;
  float* yn = y + (n * n_tokens) * v_tok + (int64_t)h * S + row0;
  float* sp = state + head * (int64_t)S * S + (int64_t)row0 * S;
  const int trow = wv * 16 + l16;                     // this lane's A-operand row
  const int last_tok = n_tokens - 1;
  // Positions past the end read the last valid row instead, unzeroed: their
  // beta and their columns of X are exactly zero, so K and V rows there meet
  // only zeros, and q rows only reach y rows that are not stored. (Zeroing
  // on load would make the compiler wait for each prefetch as it is issued.)
  auto tok_clamp = [&](int t) { return t < last_tok ? t : last_tok; };

  auto unit_of = [&](int chunk) {
    return chunk_unit(const_cast<float*>(ws), head * n_chunks + chunk);
  };
  auto fetch_kv = [&](int chunk, ChunkRegs& f) {   // K, V, factors: staged through LDS
    const int t0 = chunk * C;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int fi = (j * 256 + tid) * 4, t = fi / S, col = fi % S;
      f.kst[j] = load4(kn + (int64_t)tok_clamp(t0 + t) * kq_tok + col);
    }
    f.v = load4(vn + (int64_t)tok_clamp(t0 + (tid >> 2)) * v_tok + (tid & 3) * 4);
    const ChunkUnit u = unit_of(chunk);
    f.gam = (wv == 0) ? u.gam[lane] : 0.0f;
    f.ktf = (wv == 0) ? u.ktf[lane] : 0.0f;
    f.bet = (wv == 0) ? u.bet[lane] : 0.0f;
  };
  auto fetch_q = [&](int chunk, ChunkRegs& f) {    // q row pieces
    const float* qr = qn + (int64_t)tok_clamp(chunk * C + trow) * kq_tok + 4 * g4;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.q[j] = load4(qr + 16 * j);
  };
  auto fetch_x = [&](int chunk, ChunkRegs& f) {    // X fragments
    const ChunkUnit u = unit_of(chunk);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.x[j] = load4(u.x + ((wv * 4 + j) * 64 + lane) * 4);
  };
  auto fetch_p = [&](int chunk, ChunkRegs& f) {    // P fragments
    const ChunkUnit u = unit_of(chunk);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.p[j] = load4(u.p + ((wv * 4 + j) * 64 + lane) * 4);
  };

  // state rows: LDS copy (B operand of the M^T products) and this wave's two
  // 16 x 16 column tiles in the MFMA output layout (the update accumulators),
  // taken from the LDS copy so that no global load is pending in the loop
  for (int fi = tid * 4; fi < R * S; fi += 256 * 4)
    store4(Ms + (fi / S) * kMP + fi % S, load4(sp + fi));
  __syncthreads();
  f32x4v macc[2];
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int i = 0; i < 4; ++i) macc[c2][i] = Ms[(g4 * 4 + i) * kMP + (wv * 2 + c2) * 16 + l16];

  // K, V and the factors of a chunk from registers into LDS
  auto stage = [&](const ChunkRegs& f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int fi = (j * 256 + tid) * 4;
      store4(Ks + (fi / S) * kKSP + fi % S, f.kst[j]);
    }
    store4(Vs + (tid >> 2) * kUP + (tid & 3) * 4, f.v);
    if (wv == 0) {
      Gam[lane] = f.gam;
      Ktf[lane] = f.ktf;
      Bet[lane] = f.bet;
    }
  };
  // y rows of chunk c from LDS to memory, a float4 per thread: each wave
  // writes 16 positions x 64 contiguous bytes in one instruction (a store of
  // the MFMA output layout directly would be 16 dword stores per chunk)
  auto flush_y = [&](int chunk) {
    const int r = tid >> 2, c4 = (tid & 3) * 4;
    const int t = chunk * C + r;
    if (t < n_tokens) store4(yn + (int64_t)t * v_tok + c4, load4(Ys + r * kUP + c4));
  };

  ChunkRegs f;
  fetch_kv(0, f);
  fetch_q(0, f);
  fetch_x(0, f);
  fetch_p(0, f);

  for (int chunk = 0; chunk < n_chunks; ++chunk) {
    const int nx = chunk + 1 < n_chunks ? chunk + 1 : chunk;   // last chunk: harmless re-read
    if (chunk > 0) flush_y(chunk - 1);
    // stage this chunk's K, V and factors, then start loading the next chunk's
    stage(f);
    fetch_kv(nx, f);
    __syncthreads();

    // rows 16wv..16wv+15 of K M^T and Q M^T (K from LDS, q from registers)
    f32x4v zacc = {0.f, 0.f, 0.f, 0.f}, yacc = {0.f, 0.f, 0.f, 0.f};
    const float* mr = Ms + l16 * kMP + 4 * g4;
    const float* kr = Ks + trow * kKSP + 4 * g4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 m4 = load4(mr + 16 * j);
      const float4 k4 = load4(kr + 16 * j);
      zacc = mfma4(k4.x, m4.x, zacc);
      yacc = mfma4(f.q[j].x, m4.x, yacc);
      zacc = mfma4(k4.y, m4.y, zacc);
      yacc = mfma4(f.q[j].y, m4.y, yacc);
      zacc = mfma4(k4.z, m4.z, zacc);
      yacc = mfma4(f.q[j].z, m4.z, yacc);
      zacc = mfma4(k4.w, m4.w, zacc);
      yacc = mfma4(f.q[j].w, m4.w, yacc);
    }
    fetch_q(nx, f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wv * 16 + g4 * 4 + i;   // position of output element i
      const float bt = Bet[r], gm = Gam[r];
      Zs[r * kUP + l16] = bt * Vs[r * kUP + l16] - (bt * gm) * zacc[i];
      yacc[i] *= gm;                         // diag(gamma) Q M^T
    }
    __syncthreads();

    // U rows 16wv..16wv+15 = X Z (two accumulator chains, even and odd j)
    f32x4v ua0 = {0.f, 0.f, 0.f, 0.f}, ua1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const float* z0 = Zs + (16 * j + 4 * g4) * kUP + l16;
      const float* z1 = z0 + 16 * kUP;
      ua0 = mfma4(f.x[j].x, z0[0], ua0);
      ua1 = mfma4(f.x[j + 1].x, z1[0], ua1);
      ua0 = mfma4(f.x[j].y, z0[kUP], ua0);
      ua1 = mfma4(f.x[j + 1].y, z1[kUP], ua1);
      ua0 = mfma4(f.x[j].z, z0[2 * kUP], ua0);
      ua1 = mfma4(f.x[j + 1].z, z1[2 * kUP], ua1);
      ua0 = mfma4(f.x[j].w, z0[3 * kUP], ua0);
      ua1 = mfma4(f.x[j + 1].w, z1[3 * kUP], ua1);
    }
    const f32x4v uacc = ua0 + ua1;
    fetch_x(nx, f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wv * 16 + g4 * 4 + i;
      Us[r * kUP + l16] = uacc[i];
      Uk[r * kUP + l16] = uacc[i] * Ktf[r];
    }
    __syncthreads();

    // y += P U (a second chain for odd j), into LDS for the next chunk's flush
    f32x4v yb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const float* u0 = Us + (16 * j + 4 * g4) * kUP + l16;
      const float* u1 = u0 + 16 * kUP;
      yacc = mfma4(f.p[j].x, u0[0], yacc);
      yb = mfma4(f.p[j + 1].x, u1[0], yb);
      yacc = mfma4(f.p[j].y, u0[kUP], yacc);
      yb = mfma4(f.p[j + 1].y, u1[kUP], yb);
      yacc = mfma4(f.p[j].z, u0[2 * kUP], yacc);
      yb = mfma4(f.p[j + 1].z, u1[2 * kUP], yb);
      yacc = mfma4(f.p[j].w, u0[3 * kUP], yacc);
      yb = mfma4(f.p[j + 1].w, u1[3 * kUP], yb);
    }
    yacc = yacc + yb;
    fetch_p(nx, f);
#pragma unroll
    for (int i = 0; i < 4; ++i) Ys[(wv * 16 + g4 * 4 + i) * kUP + l16] = scale * yacc[i];
    // state update of this wave's column tiles: M = gamma_C M + (diag(Ktf) U)^T K
    // (the two column tiles interleaved: two chains sharing their A operand)
    const float gam_c = Gam[C - 1];
    const int col0 = wv * 32 + l16;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int i = 0; i < 4; ++i) macc[c2][i] *= gam_c;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s0 = 16 * j + 4 * g4;
      const float* ua = Uk + s0 * kUP + l16;
      const float* kb = Ks + s0 * kKSP + col0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float a = ua[c * kUP];
        macc[0] = mfma4(a, kb[c * kKSP], macc[0]);
        macc[1] = mfma4(a, kb[c * kKSP + 16], macc[1]);
      }
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ms[(g4 * 4 + i) * kMP + col0 + 16 * c2] = macc[c2][i];
    __syncthreads();
  }
  flush_y(n_chunks - 1);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int i = 0; i < 4; ++i) sp[(g4 * 4 + i) * S + (wv * 2 + c2) * 16 + l16] = macc[c2][i];
}

}  // namespace gdn

using namespace gdn;

namespace gdn {

// Grid limits of the two chunked kernels (the preparation's blocks never
// outnumber the (sequence, V-head, chunk) units), for shapes that are
// otherwise valid; also used by the prefill before it launches anything.
int chunked_size_check(int64_t n_seqs, int64_t n_tokens, int n_v_heads) {
  const int64_t n_chunks = (n_tokens + kChC - 1) / kChC;
  const int64_t units = n_seqs * n_v_heads * n_chunks;
  const int64_t scan_blocks = n_seqs * n_v_heads * (kChS / kChR);
  if (units >= (int64_t(1) << 31) || scan_blocks >= (int64_t(1) << 31)) return GDN_ESIZE;
  return GDN_OK;
}

}  // namespace gdn

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
  if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
      !aligned16(workspace))
    return GDN_EALIGN;
  if (chunked_size_check(n_seqs, n_tokens, n_v_heads) != GDN_OK) return GDN_ESIZE;
  const int n_chunks = (n_tokens + kChC - 1) / kChC;
  // one preparation block per K-head and chunk, unless that leaves fewer than
  // four per CU: then the K-head's V-heads are split over v_groups blocks
  // (the smallest divisor of the group size that fills the chip)
  const int gq = n_v_heads / n_k_heads;
  const int64_t k_units = (int64_t)n_seqs * n_k_heads * n_chunks;
  int v_groups = 1;
  while (v_groups < gq && (gq % v_groups != 0 || k_units * v_groups < 4 * (int64_t)cu_count()))
    ++v_groups;
  const int64_t prep_blocks = k_units * v_groups;
  const int64_t scan_blocks = (int64_t)n_seqs * n_v_heads * (kChS / kChR);
  hipStream_t s = as_stream(stream);
  float* ws = reinterpret_cast<float*>(workspace);
  const int rc = launch(chunk_prep_kernel, dim3((unsigned)prep_blocks), dim3(256), 0, s, q, k, g,
                        beta, ws, n_tokens, n_k_heads, n_v_heads, n_chunks, v_groups);
  if (rc != GDN_OK) return rc;
  return launch(chunk_scan_kernel, dim3((unsigned)scan_blocks), dim3(256), 0, s, state, q, k, v,
                ws, y, n_tokens, n_k_heads, n_v_heads, n_chunks, scale);
}
