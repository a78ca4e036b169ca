/*
 * Driver of the CPU sanitizer test (tests/test_sanitize_cpu.py): built
 * together with oracle/gdn_oracle.c (the float build) under AddressSanitizer
 * and UndefinedBehaviorSanitizer, it calls every oracle routine on small
 * seeded inputs, including the edge sizes (one token, one channel, the
 * shortest and the longest conv history the oracle accepts, a ragged head
 * count), so that an out-of-bounds access or undefined behaviour in the
 * oracle fails the run. Test infrastructure only; the results are not
 * checked here (the pins do that).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef float real;
void oracle_set_threads(int n);
void oracle_decay_gate(const real *a, const real *dt_bias, const real *A_log, real *g, int n_heads,
                       long rows);
void oracle_sigmoid(const real *x, real *y, long n);
void oracle_l2norm_gqa(const real *x, real *out, long rows, int n_k_heads, int n_v_heads, int S,
                       real eps);
void oracle_conv1d_silu_seq(const real *x, const real *w, real *conv_state, real *out, int n_seqs,
                            int n_tokens, int conv_dim, int K);
void oracle_recurrence_seq(real *state, const real *q, const real *k, const real *v,
                           const real *g, const real *beta, real *y, int n_seqs, int n_tokens,
                           int n_v_heads, int S, real scale);
void oracle_gated_rmsnorm(const real *y, const real *w, const real *z, real *out, long n_rows,
                          int D, real eps);
void oracle_decode_block_bf16(const uint16_t *qkv, const uint16_t *z, const real *a,
                              const real *b, const real *conv_w, const real *A_log,
                              const real *dt_bias, const real *norm_w, real *conv_state,
                              real *state, real *out, int n_seqs, int n_k_heads, int n_v_heads,
                              int S, int K, real scale, real l2_eps, real eps);
void oracle_prefill_bf16(const uint16_t *qkv, const uint16_t *z, const real *a, const real *b,
                         const real *conv_w, const real *A_log, const real *dt_bias,
                         const real *norm_w, real *conv_state, real *state, real *out,
                         int n_seqs, int n_tokens, int n_k_heads, int n_v_heads, int S, int K,
                         real scale, real l2_eps, real eps);

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static real rnd(void) { /* splitmix64 -> uniform in [-1, 1) */
  uint64_t z = (rs += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (real)((double)(z >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

/* Exactly n elements, filled: ASan flags any read or write past them. */
static real *arr(size_t n) {
  real *p = malloc(n * sizeof(real));
  if (!p) exit(3);
  for (size_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}
static uint16_t *bits(size_t n) {
  uint16_t *p = malloc(n * sizeof(uint16_t));
  if (!p) exit(3);
  for (size_t i = 0; i < n; ++i) p[i] = (uint16_t)(0x3F00u + (unsigned)(rnd() * 255.0f + 255.0f) % 256u);
  return p;
}

static void recurrence_case(int N, int T, int H, int S) {
  const size_t nv = (size_t)N * T * H * S, ng = (size_t)N * T * H, ns = (size_t)N * H * S * S;
  real *st = arr(ns), *q = arr(nv), *k = arr(nv), *v = arr(nv), *g = arr(ng), *b = arr(ng);
  real *y = arr(nv);
  for (size_t i = 0; i < ng; ++i) g[i] = -0.5f * (g[i] + 1.0f), b[i] = 0.5f * (b[i] + 1.0f);
  oracle_recurrence_seq(st, q, k, v, g, b, y, N, T, H, S, 0.25f);
  free(st), free(q), free(k), free(v), free(g), free(b), free(y);
}

static void conv_case(int N, int T, int C, int K) {
  real *x = arr((size_t)N * T * C), *w = arr((size_t)C * K), *cs = arr((size_t)N * C * (K - 1) + 1);
  real *out = arr((size_t)N * T * C);
  oracle_conv1d_silu_seq(x, w, cs, out, N, T, C, K);
  free(x), free(w), free(cs), free(out);
}

static void block_case(int N, int T, int HK, int H, int S, int K) {
  const int C = 2 * HK * S + H * S;
  uint16_t *qkv = bits((size_t)N * T * C), *z = bits((size_t)N * T * H * S);
  real *a = arr((size_t)N * T * H), *b = arr((size_t)N * T * H), *cw = arr((size_t)C * K);
  real *al = arr(H), *dt = arr(H), *nw = arr(S), *cs = arr((size_t)N * C * (K - 1));
  real *st = arr((size_t)N * H * S * S), *out = arr((size_t)N * T * H * S);
  if (T == 1)
    oracle_decode_block_bf16(qkv, z, a, b, cw, al, dt, nw, cs, st, out, N, HK, H, S, K, 0.3f,
                             1e-6f, 1e-6f);
  oracle_prefill_bf16(qkv, z, a, b, cw, al, dt, nw, cs, st, out, N, T, HK, H, S, K, 0.3f, 1e-6f,
                      1e-6f);
  free(qkv), free(z), free(a), free(b), free(cw), free(al), free(dt), free(nw), free(cs);
  free(st), free(out);
}

int main(void) {
  for (int threads = 1; threads <= 2; ++threads) {
    oracle_set_threads(threads);
    /* gate, sigmoid, L2 norm with the repeat, gated norm */
    real *a = arr(7 * 3), *dt = arr(3), *al = arr(3), *g = arr(7 * 3);
    oracle_decay_gate(a, dt, al, g, 3, 7);
    oracle_sigmoid(a, g, 21);
    real *x = arr(5 * 2 * 12), *o = arr(5 * 6 * 12);
    oracle_l2norm_gqa(x, o, 5, 2, 6, 12, 1e-6f);
    real *y = arr(9 * 12), *w = arr(12), *z = arr(9 * 12), *out = arr(9 * 12);
    oracle_gated_rmsnorm(y, w, z, out, 9, 12, 1e-6f);
    free(a), free(dt), free(al), free(g), free(x), free(o), free(y), free(w), free(z), free(out);
    /* recurrence: one token, ragged token counts, every state size of the library */
    recurrence_case(1, 1, 1, 1);
    recurrence_case(2, 5, 3, 8);
    recurrence_case(1, 3, 2, 32);
    /* conv: K = 1 (no history), 2..4, and the longest history the oracle holds */
    conv_case(1, 1, 1, 1);
    conv_case(2, 7, 5, 2);
    conv_case(2, 3, 9, 4);
    conv_case(1, 70, 3, 65);
    /* decode layer and prefill: K = 2..4, group sizes 1 and 2 */
    block_case(2, 1, 2, 4, 8, 4);
    block_case(1, 1, 1, 1, 4, 2);
    block_case(2, 6, 2, 4, 8, 3);
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}
