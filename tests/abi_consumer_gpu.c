/*
 * The library used from plain C, with no Python and no torch: device memory
 * from hipMalloc, a stream from hipStreamCreate, and the entry points of
 * include/gdn.h. A scan with grouped queries (one full 64-token chunk and a
 * ragged tail) and a decode step with the T4 read-out are checked against
 * the oracle (test infrastructure, linked from oracle/liboracle_f32.so)
 * within |gpu - ref| <= 1e-5 + 1e-4 |ref|, and the scan's state against
 * chained decode launches bit for bit. Built by __graft_entry__.build(); run by
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

  HIP_OK(hipStreamDestroy(stream));
  printf("%d failures\n", failures);
  return failures != 0;
}
