// Gated delta-rule recurrence on gfx950: decode (one token per sequence) and
// the sequential scan (many tokens, state held in VGPRs).
//
// The rule, per (sequence, V-head, value row j) and token, is the one of
// Foundry fm_kernel_ssm.m "Delta-rule recurrence", ssm_gated_delta.cu
// Kernel 1 and mlx-native gated_delta_net_decode.metal "Mathematical
// recurrence": decay the row by exp(g), predict pred = row . k, correct by
// delta = (v_j - pred) * beta with the rank-1 update row += k * delta, and
// read out y_j = scale * (row . q) after the update.
//
// Work mapping (wave64). A state row of S floats is spread over L = S/E
// lanes, E floats per lane (gdn_device.hpp); a wave covers G = 64/L rows per
// float4 instruction. Both kernels call the same delta_rule_step with the
// same E and L, so a scan over T tokens and T decode launches produce the
// same bits. Reductions are DPP butterflies inside a 16-lane row (plus one
// ds_swizzle when L = 32): no LDS and no barrier on the per-token path.
#include "gdn_decode.hpp"
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// ---------------------------------------------------------------------------
// Short scan (n_tokens <= kShortScan): the decode kernel's layout with a token
// loop. Each wave keeps its RW rows in VGPRs for all tokens and reads k, q, v,
// g and beta of each token straight from memory (they stay in L2: every wave
// of the head reads the same 1 KiB of k and q), prefetching token t+1 while it
// computes token t. No LDS and no barrier, so a launch with many sequences and
// few tokens (a speculative-decoding verify step) streams like the decode; the
// LDS-staged scan below is for long sequences. Same step function, so the
// result equals chained decode launches bit for bit.
// ---------------------------------------------------------------------------
constexpr int kShortScan = 16;

template <int S, int RW, bool SNAP, bool T4>
__global__ __launch_bounds__(64 * kDecodeWaves) void recurrence_short_scan_kernel(
    float* __restrict__ state, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ y, float* __restrict__ snaps, int64_t n_pairs, int n_tokens,
    int n_k_heads, int n_v_heads, float scale) {
  using Lay = RecurLayout<S>;
  constexpr int E = Lay::E, L = Lay::L, G = Lay::G;
  constexpr int IT = RW / G;
  constexpr int WPH = S / RW;
  static_assert(RW % G == 0 && S % RW == 0, "rows per wave must tile the head");

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t pair = wave / WPH;   // n * H + h
  if (pair >= n_pairs) return;  // uniform across the wave; the kernel has no barrier
  const int p = lane % L;
  const int row0 = (int)(wave % WPH) * RW + lane / L;
  const int64_t n = pair / n_v_heads;
  const int h = (int)(pair % n_v_heads);
  const int kh = h % n_k_heads;
  const int64_t tok_v = (int64_t)n_v_heads * S, tok_k = (int64_t)n_k_heads * S;
  const float* qn = q + n * n_tokens * tok_k + (int64_t)kh * S;
  const float* kn = k + n * n_tokens * tok_k + (int64_t)kh * S;
  const float* vn = v + n * n_tokens * tok_v + (int64_t)h * S + row0;
  float* yn = y + n * n_tokens * tok_v + (int64_t)h * S + row0;
  const float* gn = g + n * n_tokens * n_v_heads + h;
  const float* bn = beta + n * n_tokens * n_v_heads + h;

  float* sp = state + pair * (int64_t)S * S;
  float r[IT][E];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float4 raw[E / 4];
#pragma unroll
    for (int m = 0; m < E / 4; ++m)
      raw[m] = load4_stream(sp + (int64_t)(row0 + it * G) * S + 4 * (p + L * m));
    unpack<E>(raw, r[it]);
  }

  float kk[E], qq[E], vv[IT], gg, bb;
  float4 k4 = make_float4(0.f, 0.f, 0.f, 0.f), q4 = k4;   // T4: k, q in qk_dot's layout
  const int i4 = 4 * (lane % (S / 4));
  auto read = [&](int t) {
    load_row_part<E, L>(kn + t * tok_k, p, kk);
    load_row_part<E, L>(qn + t * tok_k, p, qq);
    if constexpr (T4) {
      k4 = load4(kn + t * tok_k + i4);
      q4 = load4(qn + t * tok_k + i4);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) vv[it] = vn[t * tok_v + it * G];
    gg = gn[(int64_t)t * n_v_heads];
    bb = bn[(int64_t)t * n_v_heads];
  };
  read(0);
  for (int t = 0; t < n_tokens; ++t) {
    float kc[E], qc[E], vc[IT];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kc[e] = kk[e];
      qc[e] = qq[e];
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) vc[it] = vv[it];
    const float d = expf(gg);
    const float b = bb;
    float qk = 0.0f;
    if constexpr (T4) qk = qk_dot<S>(k4, q4);
    if (t + 1 < n_tokens) read(t + 1);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const float yj = T4 ? delta_rule_step_t4<E, L>(r[it], kc, qc, vc[it], d, b, qk, scale)
                          : delta_rule_step<E, L>(r[it], kc, qc, vc[it], d, b, scale);
      if (p == 0) yn[t * tok_v + it * G] = yj;
      if constexpr (SNAP) {
        // snapshots: ordinary stores (measured 6% faster here than streaming
        // ones; a verify step reads one of them back soon after)
        float* sn = snaps + ((n * n_tokens + t) * n_v_heads + h) * (int64_t)S * S +
                    (int64_t)(row0 + it * G) * S;
#pragma unroll
        for (int m = 0; m < E / 4; ++m)
          store4(sn + 4 * (p + L * m), make_float4(r[it][4 * m], r[it][4 * m + 1],
                                                   r[it][4 * m + 2], r[it][4 * m + 3]));
      }
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int m = 0; m < E / 4; ++m)
      store4_stream(sp + (int64_t)(row0 + it * G) * S + 4 * (p + L * m),
                    make_float4(r[it][4 * m], r[it][4 * m + 1], r[it][4 * m + 2], r[it][4 * m + 3]));
}

template <int S, bool SNAP, bool T4>
static int launch_short_scan(float* state, const float* q, const float* k, const float* v,
                             const float* g, const float* beta, float* y, float* snaps, int n_seqs,
                             int n_tokens, int n_k_heads, int n_v_heads, float scale,
                             hipStream_t stream) {
  constexpr int RW = DecodeCfg<S>::RW;
  const int64_t n_pairs = (int64_t)n_seqs * n_v_heads;
  const unsigned blocks = grid_for(n_pairs * (S / RW), kDecodeWaves);
  return launch(recurrence_short_scan_kernel<S, RW, SNAP, T4>, dim3(blocks),
                dim3(64 * kDecodeWaves), 0, stream, state, q, k, v, g, beta, y, snaps, n_pairs,
                n_tokens, n_k_heads, n_v_heads, scale);
}

// ---------------------------------------------------------------------------
// Scan: a block of W waves owns R = W*G consecutive rows of one (sequence,
// head) and carries them in VGPRs through all tokens. Per chunk of CT tokens
// (64 or 32, chosen by the grid below; 16 at S = 256, where LDS is the limit)
// the block stages k and q of its head, v of its rows, and exp(g) and beta
// into LDS; the next chunk's global loads are issued before the current chunk
// is computed and land in the other LDS buffer, so there is one barrier per
// chunk and none per token. exp(g) is evaluated once per token per block (by
// the staging thread), not once per lane. A full chunk is unrolled, so every
// LDS read has an immediate offset and the next token's reads are scheduled
// under the current token's arithmetic; y goes to its own LDS array (which
// no read of the chunk can alias) and is written to HBM once per chunk.
//
// Block order: the BPH blocks of one head read the same k and q, so they are
// numbered to land on the same XCD (the hardware deals consecutive block ids
// round-robin over the 8 XCDs) and share that XCD's L2.
//
// V-head h reads K-head h mod n_k_heads of q and k (q, k are [N][T][HK][S]).
// With SNAP, the state after every token is also written to
// snaps[N][T][H][S][S] (the state layout, one image per token): a caller that
// accepts only the first M of T speculative tokens restores image M-1
// (ssm_gated_delta.cu fc_ssm_recurrence_seq, "snaps").
// ---------------------------------------------------------------------------
// Tokens per chunk: 64 while the grid fits one block per CU (the double
// buffer then takes most of the LDS); 32 when there are more blocks than CUs,
// which halves the LDS so that two blocks share a CU (measured 1.5x faster at
// 2 and 4 sequences of 4096 tokens, 2% slower at 1). S = 256 uses 16 (LDS).
template <int S, bool LONG_CHUNK>
struct ScanCfg {
  using Lay = RecurLayout<S>;
  static constexpr int W = (S / Lay::G) < 4 ? (S / Lay::G) : 4;  // waves per block
  static constexpr int R = W * Lay::G;                            // rows per block
  static constexpr int BPH = S / R;                               // blocks per head
  static constexpr int CT = S >= 256 ? 16 : (LONG_CHUNK ? 64 : 32);  // tokens per chunk
  static constexpr int THREADS = 64 * W;
  // LDS words of one chunk buffer: k, q [CT][S], v [CT][R], decay, beta, k . q [CT]
  static constexpr int KQ = CT * S;
  static constexpr int VOFF = 2 * KQ;
  static constexpr int DOFF = VOFF + CT * R;
  static constexpr int BOFF = DOFF + CT;
  static constexpr int QOFF = BOFF + CT;   // k . q per token (the T4 read-out)
  static constexpr int BUF = QOFF + CT;
  // float4 loads of k and q per thread per chunk (each of k and q)
  static constexpr int KQ4 = KQ / 4 / THREADS;
  static constexpr int VPT = (CT * R + THREADS - 1) / THREADS;    // v loads per thread
  static_assert(KQ % (4 * THREADS) == 0, "k/q chunk must split evenly into float4 per thread");
  static_assert(CT <= THREADS, "one staging thread per token");
};

template <int S, bool LONG_CHUNK, bool SNAP, bool T4>
__global__ __launch_bounds__((ScanCfg<S, LONG_CHUNK>::THREADS)) __attribute__((amdgpu_waves_per_eu(1, 2)))
void recurrence_scan_kernel(
    float* __restrict__ state, const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ y, float* __restrict__ snaps, int n_tokens, int n_k_heads,
    int n_v_heads, float scale) {
  using Lay = RecurLayout<S>;
  using Cfg = ScanCfg<S, LONG_CHUNK>;
  constexpr int E = Lay::E, L = Lay::L, G = Lay::G;
  constexpr int CT = Cfg::CT, R = Cfg::R, KQ = Cfg::KQ, BUF = Cfg::BUF, THREADS = Cfg::THREADS;
  __shared__ float smem[2 * BUF];
  __shared__ float ysm[CT * R];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int p = lane % L;
  const unsigned blk = xcd_group(blockIdx.x, gridDim.x);
  const int64_t head = blk / Cfg::BPH;                 // n * H + h
  const int rblk = (int)(blk % Cfg::BPH) * R;           // first row of the block
  const int64_t n = head / n_v_heads;
  const int h = (int)(head % n_v_heads);
  const int lrow = wv * G + lane / L;                   // row within the block
  const int row = rblk + lrow;

  const int64_t tok_stride = (int64_t)n_v_heads * S;     // v/y stride per token
  const int64_t kq_stride = (int64_t)n_k_heads * S;      // q/k stride per token
  const int64_t base_n = n * (int64_t)n_tokens;          // token index of (n, 0)
  const int kh = h % n_k_heads;
  const float* qn = q + base_n * kq_stride + (int64_t)kh * S;
  const float* kn = k + base_n * kq_stride + (int64_t)kh * S;
  const float* vn = v + base_n * tok_stride + (int64_t)h * S + rblk;
  float* yn = y + base_n * tok_stride + (int64_t)h * S + rblk;
  const float* gn = g + base_n * n_v_heads + h;
  const float* bn = beta + base_n * n_v_heads + h;

  // Registers that carry one chunk from global memory to LDS (zeroed so that
  // the T4 sums of positions past the end read defined values; those sums
  // are not stored).
  float4 pk[Cfg::KQ4], pq[Cfg::KQ4];
#pragma unroll
  for (int i = 0; i < Cfg::KQ4; ++i) pk[i] = pq[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  float pv[Cfg::VPT];
  float pdec = 0.0f, pbeta = 0.0f;

  auto fetch = [&](int t0) {
    const int ct = min(CT, n_tokens - t0);
#pragma unroll
    for (int i = 0; i < Cfg::KQ4; ++i) {
      const int f = (i * THREADS + tid) * 4;   // float index inside [CT][S]
      const int tt = f / S, col = f % S;
      if (tt < ct) {
        pk[i] = load4(kn + (int64_t)(t0 + tt) * kq_stride + col);
        pq[i] = load4(qn + (int64_t)(t0 + tt) * kq_stride + col);
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::VPT; ++i) {
      const int f = i * THREADS + tid;         // index inside [CT][R]
      const int tt = f / R, rr = f % R;
      if (f < CT * R && tt < ct) pv[i] = vn[(int64_t)(t0 + tt) * tok_stride + rr];
    }
    if (tid < ct) {
      pdec = expf(gn[(int64_t)(t0 + tid) * n_v_heads]);
      pbeta = bn[(int64_t)(t0 + tid) * n_v_heads];
    }
  };
  auto deposit = [&](float* buf, int t0) {
    const int ct = min(CT, n_tokens - t0);
#pragma unroll
    for (int i = 0; i < Cfg::KQ4; ++i) {
      const int f = (i * THREADS + tid) * 4;
      if (f / S < ct) {
        store4(buf + f, pk[i]);
        store4(buf + KQ + f, pq[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < Cfg::VPT; ++i) {
      const int f = i * THREADS + tid;
      if (f < CT * R && f / R < ct) buf[Cfg::VOFF + f] = pv[i];
    }
    if (tid < ct) {
      buf[Cfg::DOFF + tid] = pdec;
      buf[Cfg::BOFF + tid] = pbeta;
    }
    // T4: k . q of each token. The S/4 consecutive threads that hold a
    // token's k and q pieces form an aligned group with entries 4i..4i+3 in
    // its thread i: qk_dot's layout, so the value equals the decode's.
    if constexpr (T4) {
#pragma unroll
      for (int i = 0; i < Cfg::KQ4; ++i) {
        const int f = (i * THREADS + tid) * 4;
        const float qk = qk_dot<S>(pk[i], pq[i]);
        if (f % S == 0 && f / S < ct) buf[Cfg::QOFF + f / S] = qk;
      }
    }
  };

  float r[E];
  float* srow = state + head * (int64_t)S * S + (int64_t)row * S;
  load_row_part<E, L>(srow, p, r);
  // snapshot of token t: snaps[((n*T + t)*H + h)*S*S + row*S + ...]
  float* snap_row = SNAP ? snaps + (base_n * n_v_heads + h) * (int64_t)S * S + (int64_t)row * S
                         : nullptr;
  const int64_t snap_stride = (int64_t)n_v_heads * S * S;
  auto snapshot = [&](int t) {
    if constexpr (SNAP) {
#pragma unroll
      for (int m = 0; m < E / 4; ++m)
        store4_stream(snap_row + t * snap_stride + 4 * (p + L * m),
                      make_float4(r[4 * m], r[4 * m + 1], r[4 * m + 2], r[4 * m + 3]));
    }
  };

  // One token of the chunk in buffer `buf`; y goes to ysm (every lane of the
  // row writes the same value).
  auto token = [&](const float* buf, int tt) {
    float kk[E], qq[E];
    load_row_part<E, L>(buf + tt * S, p, kk);
    load_row_part<E, L>(buf + KQ + tt * S, p, qq);
    const float vj = buf[Cfg::VOFF + tt * R + lrow];
    const float d = buf[Cfg::DOFF + tt];
    const float b = buf[Cfg::BOFF + tt];
    ysm[tt * R + lrow] = T4 ? delta_rule_step_t4<E, L>(r, kk, qq, vj, d, b, buf[Cfg::QOFF + tt], scale)
                            : delta_rule_step<E, L>(r, kk, qq, vj, d, b, scale);
  };
  // A full chunk with the next token's LDS reads issued before the current
  // token's arithmetic (two register sets, rotated by the unrolled loop).
  auto full_chunk = [&](const float* buf, int t0) {
    float kk[2][E], qq[2][E], vj[2], d[2], b[2], qk[2];
    auto read = [&](int tt, int slot) {
      load_row_part<E, L>(buf + tt * S, p, kk[slot]);
      load_row_part<E, L>(buf + KQ + tt * S, p, qq[slot]);
      vj[slot] = buf[Cfg::VOFF + tt * R + lrow];
      d[slot] = buf[Cfg::DOFF + tt];
      b[slot] = buf[Cfg::BOFF + tt];
      qk[slot] = T4 ? buf[Cfg::QOFF + tt] : 0.0f;
    };
    read(0, 0);
#pragma unroll
    for (int tt = 0; tt < CT; ++tt) {
      const int cur = tt & 1;
      if (tt + 1 < CT) read(tt + 1, cur ^ 1);
      ysm[tt * R + lrow] =
          T4 ? delta_rule_step_t4<E, L>(r, kk[cur], qq[cur], vj[cur], d[cur], b[cur], qk[cur], scale)
             : delta_rule_step<E, L>(r, kk[cur], qq[cur], vj[cur], d[cur], b[cur], scale);
      snapshot(t0 + tt);
    }
  };

  fetch(0);
  deposit(smem, 0);
  __syncthreads();

  int buf_id = 0;
  for (int t0 = 0; t0 < n_tokens; t0 += CT) {
    const int ct = min(CT, n_tokens - t0);
    const bool more = t0 + CT < n_tokens;
    if (more) fetch(t0 + CT);
    const float* buf = smem + buf_id * BUF;
    if (ct == CT) {
      full_chunk(buf, t0);
    } else {
      for (int tt = 0; tt < ct; ++tt) {
        token(buf, tt);
        snapshot(t0 + tt);
      }
    }
    if (more) deposit(smem + (buf_id ^ 1) * BUF, t0 + CT);
    __syncthreads();
    // y of this chunk: R contiguous floats per token
    for (int i = tid; i < ct * R; i += THREADS) {
      const int tt = i / R, rr = i % R;
      yn[(int64_t)(t0 + tt) * tok_stride + rr] = ysm[i];
    }
    __syncthreads();
    buf_id ^= 1;
  }

#pragma unroll
  for (int m = 0; m < E / 4; ++m)
    store4(srow + 4 * (p + L * m), make_float4(r[4 * m], r[4 * m + 1], r[4 * m + 2], r[4 * m + 3]));
}

template <int S, bool SNAP, bool T4>
static int launch_scan(float* state, const float* q, const float* k, const float* v,
                       const float* g, const float* beta, float* y, float* snaps, int n_seqs,
                       int n_tokens, int n_k_heads, int n_v_heads, float scale, hipStream_t stream) {
  if (n_tokens <= kShortScan)
    return launch_short_scan<S, SNAP, T4>(state, q, k, v, g, beta, y, snaps, n_seqs, n_tokens,
                                          n_k_heads, n_v_heads, scale, stream);
  using CfgL = ScanCfg<S, true>;
  using CfgS = ScanCfg<S, false>;
  static_assert(CfgL::BPH == CfgS::BPH && CfgL::THREADS == CfgS::THREADS, "same grid either way");
  const int64_t blocks = (int64_t)n_seqs * n_v_heads * CfgL::BPH;
  if (blocks <= cu_count())
    return launch(recurrence_scan_kernel<S, true, SNAP, T4>, dim3((unsigned)blocks),
                  dim3(CfgL::THREADS), 0, stream, state, q, k, v, g, beta, y, snaps, n_tokens,
                  n_k_heads, n_v_heads, scale);
  return launch(recurrence_scan_kernel<S, false, SNAP, T4>, dim3((unsigned)blocks),
                dim3(CfgS::THREADS), 0, stream, state, q, k, v, g, beta, y, snaps, n_tokens,
                n_k_heads, n_v_heads, scale);
}

// Array sizes and grid limits of the decode and scan kernels, for shapes that
// are otherwise valid (also used by the prefill before it launches anything).
int recurrence_size_check(int64_t n_seqs, int64_t n_tokens, int n_v_heads, int state_size) {
  int64_t pairs, st, vec;
  if (!mul_ok(n_seqs, n_v_heads, &pairs) || !mul_ok(pairs, (int64_t)state_size * state_size, &st) ||
      !mul_ok(pairs * n_tokens, state_size, &vec))
    return GDN_ESIZE;
  if (pairs * (state_size / 8) / kDecodeWaves >= (int64_t(1) << 31)) return GDN_ESIZE;  // grid limit
  return GDN_OK;
}

static int check_recurrence(float* state, const float* q, const float* k, const float* v,
                            const float* g, const float* beta, float* y, int n_seqs,
                            int n_tokens, int n_k_heads, int n_v_heads, int state_size) {
  if (n_seqs < 0 || n_tokens < 0 || n_k_heads <= 0 || n_v_heads <= 0 || state_size <= 0)
    return GDN_ESIZE;
  if (n_v_heads % n_k_heads != 0) return GDN_ESIZE;
  if (!is_state_size(state_size)) return GDN_EUNSUPPORTED;
  if (n_seqs == 0 || n_tokens == 0) return kNothingToDo;
  if (!state || !q || !k || !v || !g || !beta || !y) return GDN_ENULL;
  if (recurrence_size_check(n_seqs, n_tokens, n_v_heads, state_size) != GDN_OK) return GDN_ESIZE;
  if (!aligned16(state) || !aligned16(q) || !aligned16(k)) return GDN_EALIGN;
  return GDN_OK;
}

template <bool T4>
static int dispatch_decode(float* state, const float* q, const float* k, const float* v,
                           const float* g, const float* beta, float* y, int n_seqs,
                           int n_k_heads, int n_v_heads, int state_size, float scale,
                           hipStream_t s) {
  switch (state_size) {
    case 32: return launch_decode<32, T4>(state, q, k, v, g, beta, y, n_seqs, n_k_heads, n_v_heads, scale, s);
    case 64: return launch_decode<64, T4>(state, q, k, v, g, beta, y, n_seqs, n_k_heads, n_v_heads, scale, s);
    case 128: return launch_decode<128, T4>(state, q, k, v, g, beta, y, n_seqs, n_k_heads, n_v_heads, scale, s);
    case 256: return launch_decode<256, T4>(state, q, k, v, g, beta, y, n_seqs, n_k_heads, n_v_heads, scale, s);
  }
  return GDN_EUNSUPPORTED;
}

template <bool SNAP, bool T4>
static int dispatch_scan(float* state, const float* q, const float* k, const float* v,
                         const float* g, const float* beta, float* y, float* snaps, int n_seqs,
                         int n_tokens, int n_k_heads, int n_v_heads, int state_size, float scale,
                         hipStream_t s) {
  switch (state_size) {
    case 32: return launch_scan<32, SNAP, T4>(state, q, k, v, g, beta, y, snaps, n_seqs, n_tokens, n_k_heads, n_v_heads, scale, s);
    case 64: return launch_scan<64, SNAP, T4>(state, q, k, v, g, beta, y, snaps, n_seqs, n_tokens, n_k_heads, n_v_heads, scale, s);
    case 128: return launch_scan<128, SNAP, T4>(state, q, k, v, g, beta, y, snaps, n_seqs, n_tokens, n_k_heads, n_v_heads, scale, s);
    case 256: return launch_scan<256, SNAP, T4>(state, q, k, v, g, beta, y, snaps, n_seqs, n_tokens, n_k_heads, n_v_heads, scale, s);
  }
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn

using namespace gdn;

extern "C" int gdn_recurrence(float* state, const float* q, const float* k, const float* v,
                              const float* g, const float* beta, float* y, int n_seqs,
                              int n_v_heads, int state_size, float scale, void* stream) {
  const int rc = check_recurrence(state, q, k, v, g, beta, y, n_seqs, 1, n_v_heads, n_v_heads,
                                  state_size);
  if (rc != GDN_OK) return finish_check(rc);
  return dispatch_decode<false>(state, q, k, v, g, beta, y, n_seqs, n_v_heads, n_v_heads,
                                state_size, scale, as_stream(stream));
}

extern "C" int gdn_recurrence_ex(float* state, const float* q, const float* k, const float* v,
                                 const float* g, const float* beta, float* y, int n_seqs,
                                 int n_k_heads, int n_v_heads, int state_size, float scale,
                                 int variant, void* stream) {
  if (variant != GDN_RECUR_EXACT && variant != GDN_RECUR_T4) return GDN_EUNSUPPORTED;
  const int rc = check_recurrence(state, q, k, v, g, beta, y, n_seqs, 1, n_k_heads, n_v_heads,
                                  state_size);
  if (rc != GDN_OK) return finish_check(rc);
  hipStream_t s = as_stream(stream);
  if (variant == GDN_RECUR_T4)
    return dispatch_decode<true>(state, q, k, v, g, beta, y, n_seqs, n_k_heads, n_v_heads,
                                 state_size, scale, s);
  return dispatch_decode<false>(state, q, k, v, g, beta, y, n_seqs, n_k_heads, n_v_heads,
                                state_size, scale, s);
}

extern "C" int gdn_recurrence_seq(float* state, const float* q, const float* k, const float* v,
                                  const float* g, const float* beta, float* y, int n_seqs,
                                  int n_tokens, int n_v_heads, int state_size, float scale,
                                  void* stream) {
  const int rc = check_recurrence(state, q, k, v, g, beta, y, n_seqs, n_tokens, n_v_heads,
                                  n_v_heads, state_size);
  if (rc != GDN_OK) return finish_check(rc);
  return dispatch_scan<false, false>(state, q, k, v, g, beta, y, nullptr, n_seqs, n_tokens,
                                     n_v_heads, n_v_heads, state_size, scale, as_stream(stream));
}

extern "C" int gdn_recurrence_seq_ex(float* state, const float* q, const float* k,
                                     const float* v, const float* g, const float* beta, float* y,
                                     float* snaps, int n_seqs, int n_tokens, int n_k_heads,
                                     int n_v_heads, int state_size, float scale, int variant,
                                     void* stream) {
  if (variant != GDN_RECUR_EXACT && variant != GDN_RECUR_T4) return GDN_EUNSUPPORTED;
  const int rc = check_recurrence(state, q, k, v, g, beta, y, n_seqs, n_tokens, n_k_heads,
                                  n_v_heads, state_size);
  if (rc != GDN_OK) return finish_check(rc);
  if (snaps && !aligned16(snaps)) return GDN_EALIGN;
  int64_t snap_elems;
  if (snaps && !mul_ok((int64_t)n_seqs * n_tokens * n_v_heads, (int64_t)state_size * state_size,
                       &snap_elems))
    return GDN_ESIZE;
  hipStream_t s = as_stream(stream);
  const bool t4 = variant == GDN_RECUR_T4;
  if (snaps)
    return t4 ? dispatch_scan<true, true>(state, q, k, v, g, beta, y, snaps, n_seqs, n_tokens,
                                          n_k_heads, n_v_heads, state_size, scale, s)
              : dispatch_scan<true, false>(state, q, k, v, g, beta, y, snaps, n_seqs, n_tokens,
                                           n_k_heads, n_v_heads, state_size, scale, s);
  return t4 ? dispatch_scan<false, true>(state, q, k, v, g, beta, y, nullptr, n_seqs, n_tokens,
                                         n_k_heads, n_v_heads, state_size, scale, s)
            : dispatch_scan<false, false>(state, q, k, v, g, beta, y, nullptr, n_seqs, n_tokens,
                                          n_k_heads, n_v_heads, state_size, scale, s);
}
