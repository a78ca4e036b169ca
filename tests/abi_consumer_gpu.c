/*
 * The library used from plain C, with no Python and no torch: device memory
 * from hipMalloc, a stream from hipStreamCreate, and the entry points of
 * include/gdn.h. A scan with grouped queries (one full 64-token chunk and a
 * ragged tail) and a decode step with the T4 read-out are checked against
 * the oracle (test infrastructure, linked from oracle/liboracle_f32.so)
 * within |gpu - ref| <= 1e-5 + 1e-4 |ref|, and the scan's state against
 * chained decode launches bit for bit. The decode step from raw inputs is
 * checked against its four stand-alone kernels, and the fused bf16 layer split
 * over 64-row workgroups against the one-workgroup layer, bit for bit, with
 * the split layer's workspace zeroed once by hipMemset and checked to be zero
 * again after each call. Built by __graft_entry__.build(); run by
 * tests/test_c_gpu.py. Exit status 0 means every check passed.
 *
 * Inputs are seeded draws from splitmix64 (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", 2014) with Box-Muller normals,
 * in the workloads' distributions: q, k ~ N(0, 1) normalised per head,
 * v ~ N(0, 1), g = -0.5 u, beta = u with u ~ U(0, 1), state ~ N(0, 0.05).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gdn.h"

/* the oracle's fp32 build (oracle/gdn_oracle.c) */
void oracle_recurrence_seq(float *state, const float *q, const float *k, const float *v,
                           const float *g, const float *beta, float *y, int n_seqs,
                           int n_tokens, int n_v_heads, int S, float scale);
void oracle_set_threads(int n);

static uint64_t rng_state;

static uint64_t splitmix64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static double uniform01(void) { return ((splitmix64() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

static float normal(void) {
  const double u1 = uniform01(), u2 = uniform01();
  return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static int failures = 0;

#define HIP_OK(call)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess) {                                                              \
      printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__);      \
      exit(2);                                                                           \
    }                                                                                    \
  } while (0)

#define GDN_OK_CALL(call)                                                                \
  do {                                                                                   \
    int rc_ = (call);                                                                    \
    if (rc_ != GDN_OK) {                                                                 \
      printf("%s returned %d (%s)\n", #call, rc_, gdn_strerror(rc_));                    \
      exit(3);                                                                           \
    }                                                                                    \
  } while (0)

static void close_to(const char *what, const float *got, const float *ref, size_t n) {
  size_t bad = 0, worst = 0;
  double worst_err = -1.0;
  for (size_t i = 0; i < n; ++i) {
    const double err = fabs((double)got[i] - (double)ref[i]);
    if (!(err <= 1e-5 + 1e-4 * fabs((double)ref[i]))) {
      ++bad;
      if (!(err <= worst_err)) worst_err = err, worst = i;
    }
  }
  if (bad) {
    printf("FAIL %s: %zu of %zu out of tolerance, worst at %zu: gpu %.9g ref %.9g\n", what, bad,
           n, worst, got[worst], ref[worst]);
    ++failures;
  } else {
    printf("ok   %s (%zu values)\n", what, n);
  }
}

static void same_bits(const char *what, const float *a, const float *b, size_t n) {
  if (memcmp(a, b, n * sizeof(float)) != 0) {
    printf("FAIL %s: not bit for bit\n", what);
    ++failures;
  } else {
    printf("ok   %s (bit for bit)\n", what);
  }
}

static float *dev_copy(const float *host, size_t n) {
  float *d = NULL;
  HIP_OK(hipMalloc((void **)&d, n * sizeof(float)));
  if (host) HIP_OK(hipMemcpy(d, host, n * sizeof(float), hipMemcpyHostToDevice));
  return d;
}

static void to_host(float *host, const float *d, size_t n) {
  HIP_OK(hipMemcpy(host, d, n * sizeof(float), hipMemcpyDeviceToHost));
}

/* q or k [N][T][HK][S], unit norm per head */
static void unit_rows(float *x, size_t rows, int S) {
  for (size_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int i = 0; i < S; ++i) {
      x[r * S + i] = normal();
      ss += (double)x[r * S + i] * x[r * S + i];
    }
    const float inv = (float)(1.0 / sqrt(ss));
    for (int i = 0; i < S; ++i) x[r * S + i] *= inv;
  }
}

/* repeat [N][T][HK][S] to [N][T][H][S] by index (V-head h reads K-head h mod HK) */
static void repeat_heads(float *out, const float *in, size_t nt, int HK, int H, int S) {
  for (size_t r = 0; r < nt; ++r)
    for (int h = 0; h < H; ++h)
      memcpy(out + (r * H + h) * S, in + (r * HK + h % HK) * S, sizeof(float) * S);
}

/* fp32 -> bf16 bit pattern, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static void *dev_bytes(const void *host, size_t bytes) {
  void *d = NULL;
  HIP_OK(hipMalloc(&d, bytes));
  if (host) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void all_zero(const char *what, const void *d, size_t bytes) {
  unsigned char *h = malloc(bytes);
  if (!h) exit(4);
  HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  size_t nz = 0;
  for (size_t i = 0; i < bytes; ++i) nz += h[i] != 0;
  if (nz) {
    printf("FAIL %s: %zu nonzero bytes\n", what, nz);
    ++failures;
  } else {
    printf("ok   %s\n", what);
  }
  free(h);
}

/* The decode step from raw inputs against its stand-alone kernels, and the
 * split fused layer against the one-workgroup layer: 3 sequences, 2 -> 4
 * heads, S = 128, conv width 4, two chained calls. */
static void fused_paths(hipStream_t stream) {
  const int N = 3, HK = 2, H = 4, S = 128, K = 4, C = 2 * HK * S + H * S;
  const float scale = 1.0f / sqrtf((float)S), eps = 1e-6f;
  const size_t nst = (size_t)N * H * S * S, nkq = (size_t)N * HK * S, nv = (size_t)N * H * S;
  float *st0 = malloc(nst * 4), *a = malloc((size_t)N * H * 4), *b = malloc((size_t)N * H * 4);
  float *A_log = malloc((size_t)H * 4), *dt_bias = malloc((size_t)H * 4), *qr = malloc(nkq * 4);
  float *kr = malloc(nkq * 4), *v = malloc(nv * 4), *conv_w = malloc((size_t)C * K * 4);
  float *norm_w = malloc((size_t)S * 4), *cs0 = malloc((size_t)N * C * (K - 1) * 4);
  uint16_t *qkv = malloc((size_t)N * C * 2), *z = malloc(nv * 2);
  float *h1 = malloc(nst * 4), *h2 = malloc(nst * 4);
  if (!st0 || !a || !b || !A_log || !dt_bias || !qr || !kr || !v || !conv_w || !norm_w || !cs0 ||
      !qkv || !z || !h1 || !h2)
    exit(4);
  for (size_t i = 0; i < nst; ++i) st0[i] = 0.05f * normal();
  for (int i = 0; i < N * H; ++i) a[i] = normal(), b[i] = normal();
  for (int i = 0; i < H; ++i) A_log[i] = normal(), dt_bias[i] = 0.5f * normal();
  for (size_t i = 0; i < nkq; ++i) qr[i] = normal(), kr[i] = normal();
  for (size_t i = 0; i < nv; ++i) v[i] = normal(), z[i] = to_bf16(normal());
  for (int i = 0; i < C * K; ++i) conv_w[i] = 0.5f * normal();
  for (int i = 0; i < S; ++i) norm_w[i] = 1.0f + 0.1f * normal();
  for (int i = 0; i < N * C * (K - 1); ++i) cs0[i] = normal();
  for (int i = 0; i < N * C; ++i) qkv[i] = to_bf16(normal());

  /* decode step: one launch against l2norm (q, k) + gate + sigmoid + recurrence */
  float *d_st1 = dev_copy(st0, nst), *d_st2 = dev_copy(st0, nst);
  float *d_qr = dev_copy(qr, nkq), *d_kr = dev_copy(kr, nkq), *d_v = dev_copy(v, nv);
  float *d_a = dev_copy(a, (size_t)N * H), *d_b = dev_copy(b, (size_t)N * H);
  float *d_Al = dev_copy(A_log, (size_t)H), *d_dt = dev_copy(dt_bias, (size_t)H);
  GDN_OK_CALL(gdn_ssm_a(d_Al, d_Al, H, stream)); /* in place: d_Al now holds ssm_a = -exp(A_log) */
  float *d_y1 = dev_copy(NULL, nv), *d_y2 = dev_copy(NULL, nv);
  float *d_q = dev_copy(NULL, nv), *d_k = dev_copy(NULL, nv);
  float *d_g = dev_copy(NULL, (size_t)N * H), *d_be = dev_copy(NULL, (size_t)N * H);
  for (int step = 0; step < 2; ++step) {
    GDN_OK_CALL(gdn_decode_step(d_st1, d_qr, d_kr, d_v, d_a, d_b, d_Al, d_dt, d_y1, N, HK, H, S,
                                scale, eps, stream));
    GDN_OK_CALL(gdn_l2norm_gqa(d_qr, d_q, N, HK, H, S, eps, stream));
    GDN_OK_CALL(gdn_l2norm_gqa(d_kr, d_k, N, HK, H, S, eps, stream));
    GDN_OK_CALL(gdn_decay_gate(d_a, d_dt, d_Al, d_g, H, N, stream));
    GDN_OK_CALL(gdn_sigmoid(d_b, d_be, (int64_t)N * H, stream));
    GDN_OK_CALL(gdn_recurrence(d_st2, d_q, d_k, d_v, d_g, d_be, d_y2, N, H, S, scale, stream));
  }
  HIP_OK(hipStreamSynchronize(stream));
  to_host(h1, d_y1, nv);
  to_host(h2, d_y2, nv);
  same_bits("decode step y = stand-alone kernels", h1, h2, nv);
  to_host(h1, d_st1, nst);
  to_host(h2, d_st2, nst);
  same_bits("decode step state = stand-alone kernels", h1, h2, nst);

  /* the fused bf16 layer: split over 64-row workgroups against one workgroup per K-head */
  const size_t ws_bytes = gdn_decode_block_workspace_bytes(N, HK, H);
  void *d_ws = dev_bytes(NULL, ws_bytes);
  HIP_OK(hipMemset(d_ws, 0, ws_bytes));
  uint16_t *d_qkv = dev_bytes(qkv, (size_t)N * C * 2), *d_z = dev_bytes(z, nv * 2);
  float *d_cw = dev_copy(conv_w, (size_t)C * K), *d_nw = dev_copy(norm_w, (size_t)S);
  float *d_cs1 = dev_copy(cs0, (size_t)N * C * (K - 1)), *d_cs2 = dev_copy(cs0, (size_t)N * C * (K - 1));
  HIP_OK(hipMemcpy(d_st1, st0, nst * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_st2, st0, nst * 4, hipMemcpyHostToDevice));
  for (int step = 0; step < 2; ++step) {
    GDN_OK_CALL(gdn_decode_block_bf16(d_qkv, d_z, d_a, d_b, d_cw, d_Al, d_dt, d_nw, d_cs1, d_st1,
                                      d_y1, N, HK, H, S, K, scale, eps, eps, stream));
    GDN_OK_CALL(gdn_decode_block_bf16_ex(d_qkv, d_z, d_a, d_b, d_cw, d_Al, d_dt, d_nw, d_cs2,
                                         d_st2, d_y2, d_ws, ws_bytes, N, HK, H, S, K, scale, eps,
                                         eps, stream));
    HIP_OK(hipStreamSynchronize(stream));
    all_zero("split layer workspace zero after the call", d_ws, ws_bytes);
  }
  to_host(h1, d_y1, nv);
  to_host(h2, d_y2, nv);
  same_bits("split layer out = one-workgroup layer", h1, h2, nv);
  to_host(h1, d_st1, nst);
  to_host(h2, d_st2, nst);
  same_bits("split layer state = one-workgroup layer", h1, h2, nst);
  to_host(h1, d_cs1, (size_t)N * C * (K - 1));
  to_host(h2, d_cs2, (size_t)N * C * (K - 1));
  same_bits("split layer conv history = one-workgroup layer", h1, h2, (size_t)N * C * (K - 1));

  void *devs[] = {d_st1, d_st2, d_qr, d_kr, d_v, d_a, d_b, d_Al, d_dt, d_y1, d_y2, d_q, d_k,
                  d_g, d_be, d_ws, d_qkv, d_z, d_cw, d_nw, d_cs1, d_cs2};
  for (size_t i = 0; i < sizeof(devs) / sizeof(devs[0]); ++i) HIP_OK(hipFree(devs[i]));
  free(st0), free(a), free(b), free(A_log), free(dt_bias), free(qr), free(kr), free(v);
  free(conv_w), free(norm_w), free(cs0), free(qkv), free(z), free(h1), free(h2);
}

int main(void) {
  const int N = 3, T = 70, HK = 2, H = 4, S = 64;
  const float scale = 1.0f / sqrtf((float)S);
  const size_t nkq = (size_t)N * T * HK * S, nv = (size_t)N * T * H * S, ng = (size_t)N * T * H;
  const size_t nst = (size_t)N * H * S * S;
  float *qh = malloc(nkq * 4), *kh = malloc(nkq * 4), *q = malloc(nv * 4), *k = malloc(nv * 4);
  float *v = malloc(nv * 4), *g = malloc(ng * 4), *beta = malloc(ng * 4), *st0 = malloc(nst * 4);
  float *y_ref = malloc(nv * 4), *st_ref = malloc(nst * 4), *y_gpu = malloc(nv * 4);
  float *st_gpu = malloc(nst * 4), *st_chain = malloc(nst * 4);
  if (!qh || !kh || !q || !k || !v || !g || !beta || !st0 || !y_ref || !st_ref || !y_gpu ||
      !st_gpu || !st_chain)
    return 4;
  rng_state = 20261202u;
  unit_rows(qh, (size_t)N * T * HK, S);
  unit_rows(kh, (size_t)N * T * HK, S);
  for (size_t i = 0; i < nv; ++i) v[i] = normal();
  for (size_t i = 0; i < ng; ++i) g[i] = (float)(-0.5 * uniform01());
  for (size_t i = 0; i < ng; ++i) beta[i] = (float)uniform01();
  for (size_t i = 0; i < nst; ++i) st0[i] = 0.05f * normal();
  repeat_heads(q, qh, (size_t)N * T, HK, H, S);
  repeat_heads(k, kh, (size_t)N * T, HK, H, S);

  oracle_set_threads(1);
  memcpy(st_ref, st0, nst * 4);
  oracle_recurrence_seq(st_ref, q, k, v, g, beta, y_ref, N, T, H, S, scale);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  float *d_qh = dev_copy(qh, nkq), *d_kh = dev_copy(kh, nkq), *d_v = dev_copy(v, nv);
  float *d_g = dev_copy(g, ng), *d_beta = dev_copy(beta, ng), *d_y = dev_copy(NULL, nv);
  float *d_st = dev_copy(st0, nst);

  /* the scan over all T tokens: one full 64-token chunk of the LDS scan and a ragged tail */
  GDN_OK_CALL(gdn_recurrence_seq_ex(d_st, d_qh, d_kh, d_v, d_g, d_beta, d_y, NULL, N, T, HK, H,
                                    S, scale, GDN_RECUR_EXACT, stream));
  HIP_OK(hipStreamSynchronize(stream));
  to_host(y_gpu, d_y, nv);
  to_host(st_gpu, d_st, nst);
  close_to("scan y", y_gpu, y_ref, nv);
  close_to("scan state", st_gpu, st_ref, nst);

  /* the same tokens as T decode launches (per-token slices of the inputs) */
  const size_t tkq = (size_t)HK * S, tv = (size_t)H * S;
  float *sl_q = malloc((size_t)N * tkq * 4), *sl_k = malloc((size_t)N * tkq * 4);
  float *sl_v = malloc((size_t)N * tv * 4), *sl_g = malloc((size_t)N * H * 4);
  float *sl_b = malloc((size_t)N * H * 4);
  if (!sl_q || !sl_k || !sl_v || !sl_g || !sl_b) return 4;
  float *d_sq = dev_copy(NULL, (size_t)N * tkq), *d_sk = dev_copy(NULL, (size_t)N * tkq);
  float *d_sv = dev_copy(NULL, (size_t)N * tv), *d_sg = dev_copy(NULL, (size_t)N * H);
  float *d_sb = dev_copy(NULL, (size_t)N * H), *d_sy = dev_copy(NULL, (size_t)N * tv);
  float *d_st2 = dev_copy(st0, nst);
  for (int t = 0; t < T; ++t) {
    for (int n = 0; n < N; ++n) {
      const size_t base = (size_t)n * T + t;
      memcpy(sl_q + n * tkq, qh + base * tkq, tkq * 4);
      memcpy(sl_k + n * tkq, kh + base * tkq, tkq * 4);
      memcpy(sl_v + n * tv, v + base * tv, tv * 4);
      memcpy(sl_g + n * H, g + base * H, (size_t)H * 4);
      memcpy(sl_b + n * H, beta + base * H, (size_t)H * 4);
    }
    HIP_OK(hipMemcpy(d_sq, sl_q, (size_t)N * tkq * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_sk, sl_k, (size_t)N * tkq * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_sv, sl_v, (size_t)N * tv * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_sg, sl_g, (size_t)N * H * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_sb, sl_b, (size_t)N * H * 4, hipMemcpyHostToDevice));
    GDN_OK_CALL(gdn_recurrence_ex(d_st2, d_sq, d_sk, d_sv, d_sg, d_sb, d_sy, N, HK, H, S, scale,
                                  GDN_RECUR_EXACT, NULL));
  }
  HIP_OK(hipDeviceSynchronize());
  to_host(st_chain, d_st2, nst);
  same_bits("scan state = chained decode launches", st_chain, st_gpu, nst);

  /* one decode step with the T4 read-out on the scan's final state */
  memcpy(st_ref, st_gpu, nst * 4);
  {
    const int t = T - 1;
    float *yq = malloc((size_t)N * tv * 4), *yr = malloc((size_t)N * tv * 4);
    float *qq = malloc((size_t)N * tv * 4), *kk = malloc((size_t)N * tv * 4);
    if (!yq || !yr || !qq || !kk) return 4;
    for (int n = 0; n < N; ++n) {
      const size_t base = (size_t)n * T + t;
      memcpy(qq + n * tv, q + base * tv, tv * 4);
      memcpy(kk + n * tv, k + base * tv, tv * 4);
    }
    oracle_recurrence_seq(st_ref, qq, kk, sl_v, sl_g, sl_b, yr, N, 1, H, S, scale);
    GDN_OK_CALL(gdn_recurrence_ex(d_st, d_sq, d_sk, d_sv, d_sg, d_sb, d_sy, N, HK, H, S, scale,
                                  GDN_RECUR_T4, stream));
    HIP_OK(hipStreamSynchronize(stream));
    to_host(yq, d_sy, (size_t)N * tv);
    to_host(st_gpu, d_st, nst);
    close_to("T4 decode y", yq, yr, (size_t)N * tv);
    close_to("T4 decode state", st_gpu, st_ref, nst);
    free(yq), free(yr), free(qq), free(kk);
  }

  /* an invalid call is rejected before anything is launched */
  if (gdn_recurrence_ex(d_st, d_sq, d_sk, d_sv, d_sg, d_sb, d_sy, N, 3, H, S, scale,
                        GDN_RECUR_EXACT, stream) != GDN_ESIZE) {
    printf("FAIL n_v_heads %% n_k_heads != 0 was not rejected\n");
    ++failures;
  }

  fused_paths(stream);

  HIP_OK(hipStreamDestroy(stream));
  printf("%d failures\n", failures);
  return failures != 0;
}
