// One decode layer of the Gated DeltaNet block fused into a single gfx950
// kernel: bf16 activations, fp32 state.
//
// Per sequence the layer runs conv1d + SiLU over all channels, splits the
// result as [q | k | v], L2-normalises q and k per K-head, repeats them to the
// V-heads by index (V-head vh reads K-head vh mod HK), computes beta = sigmoid(b)
// and the decay gate, takes one delta-rule step per state row, and applies the
// gated RMSNorm to the read-out (the decode order of ssm_gated_delta.cu's
// file header and "glue" kernels, with the tiled repeat of mlx-native
// gated_delta_net_decode.metal).
//
// Work split. One workgroup of 8 waves owns (sequence n, K-head kh) and with
// it every V-head vh = kh + r*HK (r < GQ = H/HK). The conv channels those
// heads read (q and k of kh, v of each vh) are read by no other workgroup, so
// each channel's history is rolled exactly once. The workgroup:
//   0. issues the small loads of phases 1-2 and 4 (conv, gate and norm inputs), then
//      the loads of all its state rows (GQ*S rows, 64 KiB per V-head), so
//      that the state's HBM transfer overlaps phases 1-2 (the hardware
//      counts outstanding loads in issue order: loads issued after the state
//      would have to wait for all of it);
//   1. convolves its (2 + GQ)*S channels into LDS and rolls their history;
//   2. L2-normalises q and k in LDS (waves 0 and 1); wave 2 computes beta and
//      exp(g) of the GQ V-heads;
//   3. runs the delta-rule step on its rows (each wave holds GQ*S/8 rows)
//      and writes y to LDS;
//   4. gated-RMSNorms each V-head's y with z (waves 0..GQ-1) and stores it.
// Every step uses the same device function as the stand-alone kernel of that
// step, so the layer equals the stand-alone kernels chained, bit for bit.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"
#include <mutex>

namespace gdn {

constexpr int kBlockS = 128;
constexpr int kBlockWaves = 8;

template <int GQ, int K>
__global__ __launch_bounds__(64 * kBlockWaves) void decode_block_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ z, const float* __restrict__ a,
    const float* __restrict__ b, const float* __restrict__ conv_w,
    const float* __restrict__ ssm_a, const float* __restrict__ dt_bias,
    const float* __restrict__ norm_w, float* __restrict__ conv_state, float* __restrict__ state,
    float* __restrict__ out, int n_k_heads, float scale, float l2_eps, float eps) {
  constexpr int S = kBlockS;
  using Lay = RecurLayout<S>;
  constexpr int E = Lay::E, L = Lay::L, G = Lay::G;
  constexpr int RW = GQ * S / kBlockWaves;  // state rows per wave
  constexpr int IT = RW / G;                // row groups per wave
  constexpr int NCH = (2 + GQ) * S;         // conv channels of the workgroup
  static_assert(RW % G == 0 && S % RW == 0, "a wave's rows must lie in one V-head");

  __shared__ float co[NCH];      // conv output: q | k | v[0..GQ)
  __shared__ float ys[GQ * S];   // read-out of each V-head
  __shared__ float gate_d[GQ];   // exp(g)
  __shared__ float gate_b[GQ];   // beta

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n_v_heads = GQ * n_k_heads;
  const int key_dim = n_k_heads * S;
  const int64_t C = 2 * (int64_t)key_dim + (int64_t)n_v_heads * S;
  const int kh = blockIdx.x % n_k_heads;
  const int64_t n = blockIdx.x / n_k_heads;

  // 0a. inputs of the conv (channels ch = tid + ci * threads) and of the gate
  constexpr int TPB = 64 * kBlockWaves;
  constexpr int CPT = (NCH + TPB - 1) / TPB;      // conv channels per thread
  float wc[CPT][K], hist[CPT][K - 1], xv[CPT];
  float* csp[CPT];
#pragma unroll
  for (int ci = 0; ci < CPT; ++ci) {
    const int ch = tid + ci * TPB;
    if (ch < NCH) {
      const int seg = ch / S, i = ch % S;
      int64_t c;
      if (seg == 0) c = (int64_t)kh * S + i;
      else if (seg == 1) c = key_dim + (int64_t)kh * S + i;
      else c = 2 * (int64_t)key_dim + (int64_t)(kh + (seg - 2) * n_k_heads) * S + i;
#pragma unroll
      for (int u = 0; u < K; ++u) wc[ci][u] = conv_w[c * K + u];
      csp[ci] = conv_state + (n * C + c) * (K - 1);
#pragma unroll
      for (int u = 0; u < K - 1; ++u) hist[ci][u] = csp[ci][u];
      xv[ci] = bf16_to_float(qkv[n * C + c]);
    }
  }
  const bool gate_lane = (wv == 2 && lane < GQ);
  float ga = 0.0f, gdt = 0.0f, gsa = 0.0f, gb = 0.0f;
  if (gate_lane) {
    const int h = kh + lane * n_k_heads;
    ga = a[n * n_v_heads + h];
    gdt = dt_bias[h];
    gsa = ssm_a[h];
    gb = b[n * n_v_heads + h];
  }

  // 0a'. z and norm_w of the gated norm (waves 0..GQ-1, one float4 group of
  // the head's row per lane), so that phase 4 waits on no global load: the
  // next workgroup on this CU needs the slots of waves 0..GQ-1 as well
  static_assert(S / 4 <= 64, "one float4 group of a norm row per lane");
  const bool norm_lane = (wv < GQ && lane < S / 4);
  uint2 zb_pre = make_uint2(0u, 0u);
  float4 nw_pre = make_float4(0.f, 0.f, 0.f, 0.f);
  if (norm_lane) {
    const int h = kh + wv * n_k_heads;
    zb_pre = *reinterpret_cast<const uint2*>(z + (n * n_v_heads + h) * S + 4 * lane);
    nw_pre = load4(norm_w + 4 * lane);
  }

  // 0b. state rows of this wave: combined row R = wv*RW + ... over the GQ heads
  const int r_head = (wv * RW) / S;                 // which of the GQ V-heads
  const int vh = kh + r_head * n_k_heads;
  const int p = lane % L;
  const int row0 = (wv * RW) % S + lane / L;        // row j within the V-head
  float* sp = state + (n * n_v_heads + vh) * (int64_t)S * S;
  float4 raw[IT][E / 4];
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int m = 0; m < E / 4; ++m)
      raw[it][m] = load4_stream(sp + (int64_t)(row0 + it * G) * S + 4 * (p + L * m));

  // 1. conv of the workgroup's channels
#pragma unroll
  for (int ci = 0; ci < CPT; ++ci) {
    const int ch = tid + ci * TPB;
    if (ch < NCH) {
      co[ch] = conv_point<K>(xv[ci], hist[ci], wc[ci]);
#pragma unroll
      for (int u = 0; u + 1 < K - 1; ++u) csp[ci][u] = hist[ci][u + 1];
      csp[ci][K - 2] = xv[ci];
    }
  }
  __syncthreads();

  // 2. L2 norm of q (wave 0) and k (wave 1); gate and beta (wave 2)
  if (wv < 2) {
    float* x = co + wv * S;
    const float ss = row_sumsq(x, S / 4, lane);
    const float inv = inv_l2norm(ss, l2_eps);
    for (int m = lane; m < S / 4; m += 64) {
      float4 v = load4(x + 4 * m);
      v.x = v.x * inv;
      v.y = v.y * inv;
      v.z = v.z * inv;
      v.w = v.w * inv;
      store4(x + 4 * m, v);
    }
  } else if (gate_lane) {
    const float gv = decay_gate(ga, gdt, gsa);
    gate_d[lane] = expf(gv);
    gate_b[lane] = sigmoid(gb);
  }
  __syncthreads();

  // 3. delta-rule step on this wave's rows
  {
    float kk[E], qq[E];
    load_row_part<E, L>(co + S, p, kk);
    load_row_part<E, L>(co, p, qq);
    const float d = gate_d[r_head];
    const float bt = gate_b[r_head];
    const float* vv = co + (2 + r_head) * S;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float r[E];
      unpack<E>(raw[it], r);
      const int j = row0 + it * G;
      const float yj = delta_rule_step<E, L>(r, kk, qq, vv[j], d, bt, scale);
      float* rp = sp + (int64_t)j * S;
#pragma unroll
      for (int m = 0; m < E / 4; ++m)
        store4_stream(rp + 4 * (p + L * m),
                      make_float4(r[4 * m], r[4 * m + 1], r[4 * m + 2], r[4 * m + 3]));
      if (p == 0) ys[r_head * S + j] = yj;
    }
  }
  __syncthreads();

  // 4. gated RMSNorm of each V-head's read-out
  if (wv < GQ) {
    const int h = kh + wv * n_k_heads;
    const float* yr = ys + wv * S;
    const float ss = row_sumsq(yr, S / 4, lane);
    const float inv = 1.0f / sqrtf(ss / (float)S + eps);
    float* orow = out + (n * n_v_heads + h) * S;
    if (norm_lane) {
      const int m = lane;
      const float4 yv = load4(yr + 4 * m);
      const float4 wv4 = nw_pre;
      const uint2 zb = zb_pre;
      const float z0 = bf16_to_float((uint16_t)(zb.x & 0xFFFFu));
      const float z1 = bf16_to_float((uint16_t)(zb.x >> 16));
      const float z2 = bf16_to_float((uint16_t)(zb.y & 0xFFFFu));
      const float z3 = bf16_to_float((uint16_t)(zb.y >> 16));
      float4 o;
      o.x = yv.x * inv * wv4.x * silu(z0);
      o.y = yv.y * inv * wv4.y * silu(z1);
      o.z = yv.z * inv * wv4.z * silu(z2);
      o.w = yv.w * inv * wv4.w * silu(z3);
      store4(orow + 4 * m, o);
    }
  }
}

template <int GQ, int K>
static int launch_block(const uint16_t* qkv, const uint16_t* z, const float* a, const float* b,
                        const float* conv_w, const float* ssm_a, const float* dt_bias,
                        const float* norm_w, float* conv_state, float* state, float* out,
                        int n_seqs, int n_k_heads, float scale, float l2_eps, float eps,
                        hipStream_t s) {
  const int64_t blocks = (int64_t)n_seqs * n_k_heads;
  return launch(decode_block_kernel<GQ, K>, dim3((unsigned)blocks), dim3(64 * kBlockWaves),
                0, s, qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out,
                n_k_heads, scale, l2_eps, eps);
}

template <int GQ>
static int launch_block_k(int K, const uint16_t* qkv, const uint16_t* z, const float* a,
                          const float* b, const float* conv_w, const float* ssm_a,
                          const float* dt_bias, const float* norm_w, float* conv_state,
                          float* state, float* out, int n_seqs, int n_k_heads, float scale,
                          float l2_eps, float eps, hipStream_t s) {
  switch (K) {
    case 2: return launch_block<GQ, 2>(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
    case 3: return launch_block<GQ, 3>(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
    case 4: return launch_block<GQ, 4>(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
  }
  return GDN_EUNSUPPORTED;
}


// ---------------------------------------------------------------------------
// The same layer split over 64-row workgroups (gdn_decode_block_bf16_ex).
//
// A workgroup of 8 waves owns 64 state rows of one V-head (8 rows per wave,
// the batched decode kernel's shape): the GQ*S/64 workgroups of a (sequence,
// K-head) group share out the state that the single-workgroup kernel above
// holds in one workgroup, 32 KiB each, so four of them fit a CU at once and
// the state streams as in the plain decode (measured at 64 sequences x
// 16 -> 32 heads: 47.3 us per layer against 50.9 us). Every workgroup convolves and L2-normalises the
// q and k of its K-head itself (from the same old history; 256 channels, a
// few KB of L2 reads), and the conv channels of v are split by row, so each
// v channel has one owner. Two steps need the whole group or the whole head,
// and each is taken by the last workgroup to arrive at a counter in the
// caller's workspace, so no workgroup ever waits for another:
//   * the q/k history of the K-head is rolled by the last of the group's
//     workgroups to count itself; each counts itself only after its own reads
//     of that history have returned (their values were consumed before its
//     first barrier), so no read can see the rolled history;
//   * the gated norm of a V-head needs all S read-outs: each workgroup stores
//     its rows' y to out with device-coherent stores and waits for them before
//     it counts itself; the last of the head's workgroups reads the head's y
//     back with device-coherent loads and writes the normalised row. The
//     stores and loads are relaxed atomics of device scope (the sc1 bit on
//     gfx950): such a store is acknowledged only once it has reached the
//     level of the memory hierarchy that all XCDs share, and such a load
//     reads from that level, so the hand-off holds whichever XCDs the two
//     workgroups run on. (The numbering that puts a group on one XCD only
//     makes the q/k re-reads hit its L2; no result depends on it.) A
//     device-scope release fence would order the same stores, but on this
//     chip it writes back the XCD's whole L2 (measured: 1.46 ms per layer
//     against 50 us), so each wave instead waits for its own y stores with a
//     counted s_waitcnt before it counts itself.
// The last arriver resets its counter to zero, so the workspace is zero again
// when the kernel ends. The arithmetic is the single-workgroup kernel's, step
// by step and in the same order (the norm's sum of squares is row_sumsq's lane
// order), so the two kernels agree bit for bit.
// ---------------------------------------------------------------------------
constexpr int kSplitRows = 64;   // state rows per workgroup
constexpr int kSplitWaves = 8;   // 8 rows per wave

template <int GQ, int K>
__global__ __launch_bounds__(64 * kSplitWaves) void decode_block_split_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ z, const float* __restrict__ a,
    const float* __restrict__ b, const float* __restrict__ conv_w,
    const float* __restrict__ ssm_a, const float* __restrict__ dt_bias,
    const float* __restrict__ norm_w, float* __restrict__ conv_state, float* __restrict__ state,
    float* __restrict__ out, unsigned* __restrict__ counters, int64_t n_groups, int n_k_heads,
    float scale, float l2_eps, float eps) {
  constexpr int S = kBlockS;
  using Lay = RecurLayout<S>;
  constexpr int E = Lay::E, L = Lay::L, G = Lay::G;
  constexpr int RW = kSplitRows / kSplitWaves;   // rows per wave
  constexpr int IT = RW / G;                      // row groups per wave
  constexpr int CPH = S / kSplitRows;             // workgroups per V-head
  constexpr int P = GQ * CPH;                     // workgroups per (sequence, K-head)
  constexpr int NCH = 2 * S + kSplitRows;         // q and k of kh, v of the rows
  constexpr int TPB = 64 * kSplitWaves;
  static_assert(NCH <= TPB && RW % G == 0 && CPH > 1, "one channel per thread; whole row groups");
  static_assert(IT * E / 4 < 16, "the state stores must fit the vmcnt field");

  __shared__ float co[NCH];          // conv output: q | k | v of the rows
  __shared__ float zs[S], ws[S];     // silu input and weight of the head's norm
  __shared__ float gate_d, gate_b;   // exp(g), beta
  __shared__ int qk_last;

  // workgroup -> (group = n * HK + kh, part); the P parts of a group are
  // numbered onto one XCD, so the group's q/k reads after the first hit its L2
  const int64_t blk = blockIdx.x;
  const int64_t grp = (blk / (kXcds * P)) * kXcds + blk % kXcds;
  const int part = (int)((blk / kXcds) % P);
  if (grp >= n_groups) return;   // the whole workgroup, before any barrier

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n_v_heads = GQ * n_k_heads;
  const int key_dim = n_k_heads * S;
  const int64_t C = 2 * (int64_t)key_dim + (int64_t)n_v_heads * S;
  const int kh = (int)(grp % n_k_heads);
  const int64_t n = grp / n_k_heads;
  const int chunk = part % CPH;
  const int vh = kh + (part / CPH) * n_k_heads;
  const int64_t pair = n * n_v_heads + vh;
  unsigned* cnt_group = counters + grp;
  unsigned* cnt_head = counters + n_groups + pair;

  // 0. conv input of this thread's channel, gate and norm inputs, then the
  //    state rows (loads issued after the state would wait for all of it)
  float wc[K], hist[K - 1], xv = 0.0f;
  float* csp = nullptr;
  const bool conv_lane = tid < NCH;
  if (conv_lane) {
    int64_t c;
    if (tid < S) c = (int64_t)kh * S + tid;
    else if (tid < 2 * S) c = key_dim + (int64_t)kh * S + (tid - S);
    else c = 2 * (int64_t)key_dim + (int64_t)vh * S + chunk * kSplitRows + (tid - 2 * S);
#pragma unroll
    for (int u = 0; u < K; ++u) wc[u] = conv_w[c * K + u];
    csp = conv_state + (n * C + c) * (K - 1);
#pragma unroll
    for (int u = 0; u < K - 1; ++u) hist[u] = csp[u];
    xv = bf16_to_float(qkv[n * C + c]);
  }
  const bool gate_lane = (wv == 5 && lane == 0);
  float ga = 0.0f, gdt = 0.0f, gsa = 0.0f, gb = 0.0f;
  if (gate_lane) {
    ga = a[pair];
    gdt = dt_bias[vh];
    gsa = ssm_a[vh];
    gb = b[pair];
  }
  static_assert(S / 4 <= 64, "one float4 group of the norm row per lane");
  const bool norm_lane = (wv == 6 && lane < S / 4);
  uint2 zb = make_uint2(0u, 0u);
  float4 nw = make_float4(0.f, 0.f, 0.f, 0.f);
  if (norm_lane) {
    zb = *reinterpret_cast<const uint2*>(z + pair * S + 4 * lane);
    nw = load4(norm_w + 4 * lane);
  }
  const int p = lane % L;
  const int row0 = chunk * kSplitRows + wv * RW + lane / L;
  float* sp = state + pair * (int64_t)S * S;
  float4 raw[IT][E / 4];
#pragma unroll
  for (int it = 0; it < IT; ++it)
#pragma unroll
    for (int m = 0; m < E / 4; ++m)
      raw[it][m] = load4_stream(sp + (int64_t)(row0 + it * G) * S + 4 * (p + L * m));

  // 1. conv; the rows' own v channels roll their history at once
  if (conv_lane) {
    co[tid] = conv_point<K>(xv, hist, wc);
    if (tid >= 2 * S) {
#pragma unroll
      for (int u = 0; u + 1 < K - 1; ++u) csp[u] = hist[u + 1];
      csp[K - 2] = xv;
    }
  }
  if (norm_lane) {
    zs[4 * lane + 0] = bf16_to_float((uint16_t)(zb.x & 0xFFFFu));
    zs[4 * lane + 1] = bf16_to_float((uint16_t)(zb.x >> 16));
    zs[4 * lane + 2] = bf16_to_float((uint16_t)(zb.y & 0xFFFFu));
    zs[4 * lane + 3] = bf16_to_float((uint16_t)(zb.y >> 16));
    store4(ws + 4 * lane, nw);
  }
  __syncthreads();

  // 2. L2 norm of q (wave 0) and k (wave 1); gate and beta (wave 5)
  if (wv < 2) {
    float* x = co + wv * S;
    const float ss = row_sumsq(x, S / 4, lane);
    const float inv = inv_l2norm(ss, l2_eps);
    for (int m = lane; m < S / 4; m += 64) {
      float4 v = load4(x + 4 * m);
      v.x = v.x * inv;
      v.y = v.y * inv;
      v.z = v.z * inv;
      v.w = v.w * inv;
      store4(x + 4 * m, v);
    }
  } else if (gate_lane) {
    const float gv = decay_gate(ga, gdt, gsa);
    gate_d = expf(gv);
    gate_b = sigmoid(gb);
  }
  __syncthreads();

  // Every read of the group's shared q/k history by this workgroup returned
  // before the first barrier: count the workgroup. Wave 4 waits for the
  // count where it waits for its state rows anyway; the result is used after
  // the step.
  unsigned group_old = 0u;
  if (wv == 4 && lane == 0)
    group_old = __hip_atomic_fetch_add(cnt_group, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // 3. delta-rule step on this wave's rows; y is published before the state
  //    goes back
  float* yrow = out + pair * S;
  {
    float kk[E], qq[E];
    load_row_part<E, L>(co + S, p, kk);
    load_row_part<E, L>(co, p, qq);
    const float d = gate_d;
    const float bt = gate_b;
    const float* vv = co + 2 * S - chunk * kSplitRows;   // v of row j is vv[j]
    float r[IT][E];
    float yj[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      unpack<E>(raw[it], r[it]);
      yj[it] = delta_rule_step<E, L>(r[it], kk, qq, vv[row0 + it * G], d, bt, scale);
    }
    if (p == 0) {
#pragma unroll
      for (int it = 0; it < IT; ++it)
        __hip_atomic_store(yrow + row0 + it * G, yj[it], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float* rp = sp + (int64_t)(row0 + it * G) * S;
#pragma unroll
      for (int m = 0; m < E / 4; ++m)
        store4_stream(rp + 4 * (p + L * m), make_float4(r[it][4 * m], r[it][4 * m + 1],
                                                        r[it][4 * m + 2], r[it][4 * m + 3]));
    }
    // Vector memory operations complete in issue order: with the IT*E/4 state
    // stores still allowed in flight, the y stores issued before them are done.
    // The signal fences keep the compiler from moving memory operations across
    // the wait. The immediate is gfx9's s_waitcnt encoding (vmcnt in bits 3:0,
    // expcnt 6:4 and lgkmcnt 11:8 at their maxima, i.e. not waited on).
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((IT * E / 4) | (7 << 4) | (15 << 8));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
  if (wv == 4 && lane == 0) {
    qk_last = (group_old == (unsigned)(P - 1));
    if (group_old == (unsigned)(P - 1))
      __hip_atomic_store(cnt_group, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // the group's last workgroup rolls the q/k history (every other one has read it)
  if (qk_last && tid < 2 * S) {
#pragma unroll
    for (int u = 0; u + 1 < K - 1; ++u) csp[u] = hist[u + 1];
    csp[K - 2] = xv;
  }

  // 4. every wave's y has reached memory. Wave 0 counts the workgroup for its
  //    V-head; the head's last workgroup applies the gated norm to all S rows.
  if (wv != 0) return;
  unsigned head_old = 0u;
  if (lane == 0) {
    head_old = __hip_atomic_fetch_add(cnt_head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (head_old == (unsigned)(CPH - 1))
      __hip_atomic_store(cnt_head, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  head_old = __builtin_amdgcn_readfirstlane(head_old);
  if (head_old != (unsigned)(CPH - 1)) return;
  // the sum of squares in row_sumsq's order: lane m holds entries 4m..4m+3
  float y4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float ss = 0.0f;
  if (lane < S / 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      y4[e] = __hip_atomic_load(yrow + 4 * lane + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(y4[e], y4[e], ss);
  }
  ss = group_sum<64>(ss);
  const float inv = 1.0f / sqrtf(ss / (float)S + eps);
  if (lane < S / 4) {
    const float4 w4 = load4(ws + 4 * lane);
    float4 o;
    o.x = y4[0] * inv * w4.x * silu(zs[4 * lane + 0]);
    o.y = y4[1] * inv * w4.y * silu(zs[4 * lane + 1]);
    o.z = y4[2] * inv * w4.z * silu(zs[4 * lane + 2]);
    o.w = y4[3] * inv * w4.w * silu(zs[4 * lane + 3]);
    store4(yrow + 4 * lane, o);
  }
}

template <int GQ, int K>
static int launch_block_split(const uint16_t* qkv, const uint16_t* z, const float* a,
                              const float* b, const float* conv_w, const float* ssm_a,
                              const float* dt_bias, const float* norm_w, float* conv_state,
                              float* state, float* out, unsigned* counters, int64_t groups,
                              int n_k_heads, float scale, float l2_eps, float eps, hipStream_t s) {
  constexpr int P = GQ * (kBlockS / kSplitRows);
  const int64_t blocks = ((groups + kXcds - 1) / kXcds) * kXcds * P;
  return launch(decode_block_split_kernel<GQ, K>, dim3((unsigned)blocks),
                dim3(64 * kSplitWaves), 0, s, qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w,
                conv_state, state, out, counters, groups, n_k_heads, scale, l2_eps, eps);
}

template <int GQ>
static int launch_block_split_k(int K, const uint16_t* qkv, const uint16_t* z, const float* a,
                                const float* b, const float* conv_w, const float* ssm_a,
                                const float* dt_bias, const float* norm_w, float* conv_state,
                                float* state, float* out, unsigned* counters, int64_t groups,
                                int n_k_heads, float scale, float l2_eps, float eps, hipStream_t s) {
  switch (K) {
    case 2: return launch_block_split<GQ, 2>(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, counters, groups, n_k_heads, scale, l2_eps, eps, s);
    case 3: return launch_block_split<GQ, 3>(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, counters, groups, n_k_heads, scale, l2_eps, eps, s);
    case 4: return launch_block_split<GQ, 4>(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, counters, groups, n_k_heads, scale, l2_eps, eps, s);
  }
  return GDN_EUNSUPPORTED;
}

}  // namespace gdn

using namespace gdn;

extern "C" int gdn_decode_block_bf16(const uint16_t* qkv, const uint16_t* z, const float* a,
                                     const float* b, const float* conv_w, const float* ssm_a,
                                     const float* dt_bias, const float* norm_w,
                                     float* conv_state, float* state, float* out, int n_seqs,
                                     int n_k_heads, int n_v_heads, int state_size,
                                     int conv_kernel, float scale, float l2_eps, float eps,
                                     void* stream) {
  if (n_seqs < 0 || n_k_heads <= 0 || n_v_heads <= 0 || state_size <= 0 || conv_kernel <= 0)
    return GDN_ESIZE;
  if (n_v_heads % n_k_heads != 0) return GDN_ESIZE;
  const int gq = n_v_heads / n_k_heads;
  if (state_size != kBlockS || !(gq == 1 || gq == 2 || gq == 4)) return GDN_EUNSUPPORTED;
  if (conv_kernel < 2 || conv_kernel > 4) return GDN_EUNSUPPORTED;
  if (n_seqs == 0) return GDN_OK;
  if (!qkv || !z || !a || !b || !conv_w || !ssm_a || !dt_bias || !norm_w || !conv_state ||
      !state || !out)
    return GDN_ENULL;
  int64_t pairs, st;
  if (!mul_ok(n_seqs, n_v_heads, &pairs) || !mul_ok(pairs, (int64_t)state_size * state_size, &st))
    return GDN_ESIZE;
  if ((int64_t)n_seqs * n_k_heads >= (int64_t(1) << 31)) return GDN_ESIZE;
  if (!aligned16(state) || !aligned16(norm_w) || !aligned16(out)) return GDN_EALIGN;
  if ((reinterpret_cast<uintptr_t>(z) & 7u) != 0) return GDN_EALIGN;
  hipStream_t s = as_stream(stream);
  switch (gq) {
    case 1: return launch_block_k<1>(conv_kernel, qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
    case 2: return launch_block_k<2>(conv_kernel, qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
    case 4: return launch_block_k<4>(conv_kernel, qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, n_seqs, n_k_heads, scale, l2_eps, eps, s);
  }
  return GDN_EUNSUPPORTED;
}


// Counters of gdn_decode_block_bf16_ex: one per (sequence, K-head) group and
// one per (sequence, V-head).
static bool block_counters(int n_seqs, int n_k_heads, int n_v_heads, int64_t* count) {
  int64_t groups, heads;
  if (!mul_ok(n_seqs, n_k_heads, &groups) || !mul_ok(n_seqs, n_v_heads, &heads)) return false;
  *count = groups + heads;
  return true;
}

extern "C" size_t gdn_decode_block_workspace_bytes(int n_seqs, int n_k_heads, int n_v_heads) {
  if (n_seqs < 0 || n_k_heads <= 0 || n_v_heads <= 0 || n_v_heads % n_k_heads != 0) return 0;
  int64_t count;
  if (!block_counters(n_seqs, n_k_heads, n_v_heads, &count)) return 0;
  return (size_t)count * sizeof(unsigned);
}

// Argument checks of the split layer (all but the workspace's), shared by the
// workspace and the allocation-free entry points.
static int check_block_split(const uint16_t* qkv, const uint16_t* z, const float* a,
                             const float* b, const float* conv_w, const float* ssm_a,
                             const float* dt_bias, const float* norm_w, const float* conv_state,
                             const float* state, const float* out, int n_seqs, int n_k_heads,
                             int n_v_heads, int state_size, int conv_kernel, int64_t* counters) {
  if (n_seqs < 0 || n_k_heads <= 0 || n_v_heads <= 0 || state_size <= 0 || conv_kernel <= 0)
    return GDN_ESIZE;
  if (n_v_heads % n_k_heads != 0) return GDN_ESIZE;
  const int gq = n_v_heads / n_k_heads;
  if (state_size != kBlockS || !(gq == 1 || gq == 2 || gq == 4)) return GDN_EUNSUPPORTED;
  if (conv_kernel < 2 || conv_kernel > 4) return GDN_EUNSUPPORTED;
  if (n_seqs == 0) return kNothingToDo;
  if (!qkv || !z || !a || !b || !conv_w || !ssm_a || !dt_bias || !norm_w || !conv_state ||
      !state || !out)
    return GDN_ENULL;
  int64_t pairs, st;
  if (!mul_ok(n_seqs, n_v_heads, &pairs) || !mul_ok(pairs, (int64_t)state_size * state_size, &st))
    return GDN_ESIZE;
  if (!block_counters(n_seqs, n_k_heads, n_v_heads, counters)) return GDN_ESIZE;
  const int64_t groups = (int64_t)n_seqs * n_k_heads;
  const int64_t blocks = ((groups + kXcds - 1) / kXcds) * kXcds * gq * (kBlockS / kSplitRows);
  if (blocks >= (int64_t(1) << 31)) return GDN_ESIZE;
  if (!aligned16(state) || !aligned16(norm_w) || !aligned16(out)) return GDN_EALIGN;
  if ((reinterpret_cast<uintptr_t>(z) & 7u) != 0) return GDN_EALIGN;
  return GDN_OK;
}

static int dispatch_block_split(const uint16_t* qkv, const uint16_t* z, const float* a,
                                const float* b, const float* conv_w, const float* ssm_a,
                                const float* dt_bias, const float* norm_w, float* conv_state,
                                float* state, float* out, unsigned* counters, int n_seqs,
                                int n_k_heads, int n_v_heads, int conv_kernel, float scale,
                                float l2_eps, float eps, hipStream_t s) {
  const int64_t groups = (int64_t)n_seqs * n_k_heads;
  switch (n_v_heads / n_k_heads) {
    case 1: return launch_block_split_k<1>(conv_kernel, qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, counters, groups, n_k_heads, scale, l2_eps, eps, s);
    case 2: return launch_block_split_k<2>(conv_kernel, qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, counters, groups, n_k_heads, scale, l2_eps, eps, s);
    case 4: return launch_block_split_k<4>(conv_kernel, qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state, out, counters, groups, n_k_heads, scale, l2_eps, eps, s);
  }
  return GDN_EUNSUPPORTED;
}

extern "C" int gdn_decode_block_bf16_ex(const uint16_t* qkv, const uint16_t* z, const float* a,
                                        const float* b, const float* conv_w, const float* ssm_a,
                                        const float* dt_bias, const float* norm_w,
                                        float* conv_state, float* state, float* out,
                                        void* workspace, size_t workspace_bytes, int n_seqs,
                                        int n_k_heads, int n_v_heads, int state_size,
                                        int conv_kernel, float scale, float l2_eps, float eps,
                                        void* stream) {
  int64_t count = 0;
  const int rc = check_block_split(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state,
                                   state, out, n_seqs, n_k_heads, n_v_heads, state_size,
                                   conv_kernel, &count);
  if (rc != GDN_OK) return finish_check(rc);
  if (!workspace) return GDN_ENULL;
  if (workspace_bytes < (size_t)count * sizeof(unsigned)) return GDN_ESIZE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return GDN_EALIGN;
  return dispatch_block_split(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state,
                              out, static_cast<unsigned*>(workspace), n_seqs, n_k_heads,
                              n_v_heads, conv_kernel, scale, l2_eps, eps, as_stream(stream));
}

// ---------------------------------------------------------------------------
// The split layer without a workspace argument (gdn_decode_block_bf16_noalloc),
// for callers that cannot allocate device memory. Its counters live in a
// library-owned device array, one per GPU, of GDN_NOALLOC_MAX_COUNTERS 32-bit
// counters (256 KiB), held until the process ends. The array has no
// initialiser, so it starts zero on every device, and every completed call
// leaves the counters it used zero again (the split kernel's last arrivers
// reset them), so no call needs to clear it. Calls that overlap on one GPU
// share the array and race.
// ---------------------------------------------------------------------------
namespace gdn {

constexpr int64_t kNoAllocCounters = GDN_NOALLOC_MAX_COUNTERS;
static_assert(kNoAllocCounters * sizeof(unsigned) <= 256 * 1024, "a modest scratch array");

__device__ __align__(256) unsigned scratch[kNoAllocCounters];

// Device address of the current GPU's copy of `scratch`, looked up once per
// device with that device current. In host code the array's name is only a
// host-side stand-in: a kernel must be given this address, never the name.
static int scratch_address(unsigned** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<unsigned*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ELAUNCH;
  unsigned* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* sym = nullptr;
      if (hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch)) != hipSuccess || !sym) return GDN_ELAUNCH;
      p = static_cast<unsigned*>(sym);
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GDN_OK;
}

}  // namespace gdn

extern "C" int gdn_decode_block_bf16_noalloc(const uint16_t* qkv, const uint16_t* z,
                                             const float* a, const float* b,
                                             const float* conv_w, const float* ssm_a,
                                             const float* dt_bias, const float* norm_w,
                                             float* conv_state, float* state, float* out,
                                             int n_seqs, int n_k_heads, int n_v_heads,
                                             int state_size, int conv_kernel, float scale,
                                             float l2_eps, float eps, void* stream) {
  int64_t count = 0;
  const int rc = check_block_split(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state,
                                   state, out, n_seqs, n_k_heads, n_v_heads, state_size,
                                   conv_kernel, &count);
  if (rc != GDN_OK) return finish_check(rc);
  if (count > kNoAllocCounters) return GDN_ESIZE;
  unsigned* counters = nullptr;
  const int src = scratch_address(&counters);
  if (src != GDN_OK) return src;
  return dispatch_block_split(qkv, z, a, b, conv_w, ssm_a, dt_bias, norm_w, conv_state, state,
                              out, counters, n_seqs, n_k_heads, n_v_heads, conv_kernel, scale,
                              l2_eps, eps, as_stream(stream));
}
