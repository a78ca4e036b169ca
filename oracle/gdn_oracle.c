/*
 * Gated DeltaNet oracle: a plain, sequential CPU statement of what the
 * Gated DeltaNet SSM block computes.
 *
 * THIS FILE IS TEST INFRASTRUCTURE. Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load or call it. The HIP library
 * and its Python binding never link, load or call it, and it shares no code,
 * header or table with them.
 *
 * Sources. The three pages this follows are:
 *   [FM]  Foundry, metal/kernels/fm_kernel_ssm.m (Metal host dispatch + MSL)
 *   [CU]  Foundry, cuda_kernels/ssm_gated_delta.cu at commit 775df8ab
 *   [MLX] mlx-native 0.21.1, src/shaders/gated_delta_net_decode.metal
 * Each function below names the section of the page it restates.
 *
 * Precision. The pages keep the state and every scalar in IEEE fp32. This one
 * source is compiled twice:
 *   - without ORACLE_F64: `real` is float and the float libm calls are used
 *     (expf, log1pf, sqrtf). This is the parity reference.
 *   - with ORACLE_F64: `real` is double (exp, log1p, sqrt). The same steps in
 *     double precision; tests use it to bound the float build's own rounding.
 * Both are built with -ffp-contract=off, so every product and every sum is
 * rounded on its own, and every dot product is summed in ascending index order
 * starting from +0. There is no blocking, fusion or reordering: each function
 * is the definition written out.
 *
 * Parallelism. The outermost loop over independent units (rows of the state,
 * channels, normalisation rows) may run under OpenMP; that never changes the
 * arithmetic of any single unit. oracle_set_threads() fixes the thread count.
 *
 * Layouts (row-major, last index fastest):
 *   state  [N][H][S][S]    state[n][h][j][i] is entry (i, j) of the pages'
 *                          per-head state, i over the key dimension and
 *                          j over the value dimension (the transposed layout:
 *                          row j holds S contiguous values over i)
 *   q,k,v,y [N][T][H][S]   g, beta [N][T][H]
 *   conv x/out [N][T][C]   conv weight [C][K]   conv_state [N][C][K-1]
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef ORACLE_F64
typedef double real;
#define R_EXP exp
#define R_LOG1P log1p
#define R_SQRT sqrt
#define ORACLE_PRECISION_NAME "f64"
#else
typedef float real;
#define R_EXP expf
#define R_LOG1P log1pf
#define R_SQRT sqrtf
#define ORACLE_PRECISION_NAME "f32"
#endif

const char *oracle_precision(void) { return ORACLE_PRECISION_NAME; }

int oracle_real_size(void) { return (int)sizeof(real); }

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Scalar helpers
 * ------------------------------------------------------------------------ */

/* SiLU in its divisor form, x / (1 + exp(-x)): [FM] "SiLU" helper and [CU]
 * fc_ssm_silu both state this form. For x below about -88 exp(-x) overflows
 * to +inf and the result is -0; that is accepted. */
static real silu(real x)
{
    return x / ((real)1 + R_EXP(-x));
}

/* softplus(u) = log(1 + e^u), returned as u itself when u > 20 so that e^u
 * never overflows: [CU] fc_ssm_decay_gate and [FM] "Decay gate" section,
 * which gives the guard's reason (an infinite softplus would make the decay
 * exactly zero and wipe the head's state). */
static real softplus_guarded(real u)
{
    if (u > (real)20)
        return u;
    return R_LOG1P(R_EXP(u));
}

/* Logistic sigmoid 1 / (1 + e^-x): [CU] fc_sigmoid (beta's gate). */
static real sigmoid(real x)
{
    return (real)1 / ((real)1 + R_EXP(-x));
}

/* bf16 -> fp32 widening is exact: the 16 stored bits are the top half of the
 * float's bit pattern. */
static real bf16_to_real(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (real)f;
}

/* ------------------------------------------------------------------------
 * Decay gate
 *
 * [CU] fc_ssm_decay_gate / fc_ssm_decay_gate_nx and [FM] "Decay gate":
 *     g[r][h] = ssm_a[h] * softplus(a[r][h] + dt_bias[h]),
 *     ssm_a[h] = -exp(A_log[h]).
 * ssm_a is computed here from A_log (the pages pre-compute it on the host);
 * A_log and dt_bias are per head and broadcast over rows. g <= 0, so the
 * per-token decay exp(g) lies in (0, 1].
 * ------------------------------------------------------------------------ */
void oracle_decay_gate(const real *a, const real *dt_bias, const real *A_log,
                       real *g, int n_heads, long rows)
{
    for (long r = 0; r < rows; r++) {
        for (int h = 0; h < n_heads; h++) {
            real u = a[r * n_heads + h] + dt_bias[h];
            real ssm_a = -R_EXP(A_log[h]);
            g[r * n_heads + h] = ssm_a * softplus_guarded(u);
        }
    }
}

/* beta = sigmoid(b), element-wise: [CU] fc_sigmoid. */
void oracle_sigmoid(const real *x, real *y, long n)
{
    for (long e = 0; e < n; e++)
        y[e] = sigmoid(x[e]);
}

/* ------------------------------------------------------------------------
 * q/k L2 normalisation and grouped-query repeat
 *
 * [CU] fc_ssm_qknorm_gqa: each K-head vector is divided by
 * max(||x||_2, eps); V-head vh then reads K-head vh mod n_k_heads (the tiled
 * repeat vh = r * n_k_heads + kh, also [MLX] "GQA: tiled mapping").
 *   x   [rows][n_k_heads][S]
 *   out [rows][n_v_heads][S]
 * ------------------------------------------------------------------------ */
void oracle_l2norm_gqa(const real *x, real *out, long rows, int n_k_heads,
                       int n_v_heads, int S, real eps)
{
    real *xhat = (real *)malloc(sizeof(real) * (size_t)S);
    for (long r = 0; r < rows; r++) {
        for (int kh = 0; kh < n_k_heads; kh++) {
            const real *src = x + ((size_t)r * n_k_heads + kh) * S;
            real ss = 0;
            for (int i = 0; i < S; i++)
                ss = ss + src[i] * src[i];
            real norm = R_SQRT(ss);
            real inv = (real)1 / (norm > eps ? norm : eps);
            for (int i = 0; i < S; i++)
                xhat[i] = src[i] * inv;
            for (int vh = kh; vh < n_v_heads; vh += n_k_heads) {
                real *dst = out + ((size_t)r * n_v_heads + vh) * S;
                for (int i = 0; i < S; i++)
                    dst[i] = xhat[i];
            }
        }
    }
    free(xhat);
}

/* ------------------------------------------------------------------------
 * Causal depthwise conv1d + SiLU with a rolling history
 *
 * [FM] "Causal depthwise conv1d + SiLU" (fmssm_conv1d_silu and its scan
 * fmssm_conv1d_silu_seq) and [CU] Kernel 2 / fc_ssm_conv1d_silu_seq:
 * per channel c the window is the K-1 stored inputs (oldest first) followed
 * by the current input x; the weight w[c][K-1] multiplies x. The sum starts
 * from the newest tap, x * w[c][K-1], then adds hist[u] * w[c][u] for
 * u = 0 .. K-2 in ascending order; the output is SiLU of that sum. The
 * history then drops its oldest entry and appends the raw x (not the
 * convolved value). A scan over T positions equals T single steps.
 *   x, out [N][T][C], w [C][K], conv_state [N][C][K-1] (updated in place)
 * ------------------------------------------------------------------------ */
/* Longest conv history a channel may carry (the pages' widths are 2..4). */
#define ORACLE_MAX_TAPS 64

void oracle_conv1d_silu_seq(const real *x, const real *w, real *conv_state,
                            real *out, int n_seqs, int n_tokens, int conv_dim,
                            int K)
{
    const int taps = K - 1;
    if (K < 1 || taps > ORACLE_MAX_TAPS) {
        fprintf(stderr, "oracle_conv1d_silu_seq: conv_kernel %d outside 1..%d\n", K,
                ORACLE_MAX_TAPS + 1);
        abort();
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < n_seqs; n++) {
        for (int c = 0; c < conv_dim; c++) {
            real hist[ORACLE_MAX_TAPS];
            const real *wc = w + (size_t)c * K;
            real *cs = conv_state + ((size_t)n * conv_dim + c) * taps;
            for (int u = 0; u < taps; u++)
                hist[u] = cs[u];
            for (int t = 0; t < n_tokens; t++) {
                size_t idx = ((size_t)n * n_tokens + t) * conv_dim + c;
                real xv = x[idx];
                real acc = xv * wc[taps];
                for (int u = 0; u < taps; u++)
                    acc = acc + hist[u] * wc[u];
                out[idx] = silu(acc);
                for (int u = 0; u + 1 < taps; u++)
                    hist[u] = hist[u + 1];
                if (taps > 0)
                    hist[taps - 1] = xv;
            }
            for (int u = 0; u < taps; u++)
                cs[u] = hist[u];
        }
    }
}

/* ------------------------------------------------------------------------
 * Gated delta-rule recurrence
 *
 * [FM] "Delta-rule recurrence" (fmssm_recurrence, and the sequential scan
 * fmssm_recurrence_seq), [CU] Kernel 1 fc_ssm_recurrence and
 * fc_ssm_recurrence_seq, [MLX] "Mathematical recurrence". For every
 * (sequence n, V-head h, value row j), with r the stored row j of head h
 * (r[i] = entry (i, j) of the state), and for each token t in order:
 *   1. d = exp(g[n][t][h])              scalar decay, g <= 0
 *   2. r[i] = r[i] * d                  for every i
 *   3. pred = sum_i r[i] * k[i]         ascending i
 *   4. delta = (v[j] - pred) * beta[n][t][h]
 *   5. r[i] = r[i] + k[i] * delta       rank-1 update of the row
 *   6. y[j] = scale * sum_i r[i] * q[i] read AFTER the update, ascending i
 * and the row is stored back after the last token. Decode is n_tokens = 1.
 * Rows are independent of one another. q and k are the per-V-head vectors
 * (after any grouped-query repeat). [MLX] writes the decay as exp(-g) with a
 * positive g; here g is the gate's own (non-positive) output, as on [FM] and
 * [CU].
 * ------------------------------------------------------------------------ */
void oracle_recurrence_seq(real *state, const real *q, const real *k,
                           const real *v, const real *g, const real *beta,
                           real *y, int n_seqs, int n_tokens, int n_v_heads,
                           int S, real scale)
{
    const long n_rows = (long)n_seqs * n_v_heads * S;
#pragma omp parallel for schedule(static)
    for (long row = 0; row < n_rows; row++) {
        const int j = (int)(row % S);
        const int h = (int)((row / S) % n_v_heads);
        const int n = (int)(row / ((long)S * n_v_heads));
        real *r = state + (size_t)row * S;
        for (int t = 0; t < n_tokens; t++) {
            const size_t tok = (size_t)n * n_tokens + t;
            const size_t vec = (tok * n_v_heads + h) * S;
            const real d = R_EXP(g[tok * n_v_heads + h]);
            const real b = beta[tok * n_v_heads + h];
            const real *kt = k + vec;
            const real *qt = q + vec;

            for (int i = 0; i < S; i++)
                r[i] = r[i] * d;

            real pred = 0;
            for (int i = 0; i < S; i++)
                pred = pred + r[i] * kt[i];

            const real delta = (v[vec + j] - pred) * b;

            for (int i = 0; i < S; i++)
                r[i] = r[i] + kt[i] * delta;

            real o = 0;
            for (int i = 0; i < S; i++)
                o = o + r[i] * qt[i];
            y[vec + j] = scale * o;
        }
    }
}

/* ------------------------------------------------------------------------
 * Gated RMSNorm
 *
 * [FM] "Gated RMSNorm" (fmssm_gated_norm) and [CU] Kernel 3
 * fc_ssm_gated_norm: per row of D values (one V-head of one token)
 *   inv = 1 / sqrt(mean(y^2) + eps)
 *   out[d] = y[d] * inv * w[d] * silu(z[d])
 * The weight w has length D and is shared by every head.
 * ------------------------------------------------------------------------ */
void oracle_gated_rmsnorm(const real *y, const real *w, const real *z,
                          real *out, long n_rows, int D, real eps)
{
#pragma omp parallel for schedule(static)
    for (long r = 0; r < n_rows; r++) {
        const real *yr = y + (size_t)r * D;
        const real *zr = z + (size_t)r * D;
        real *o = out + (size_t)r * D;
        real ss = 0;
        for (int d = 0; d < D; d++)
            ss = ss + yr[d] * yr[d];
        const real inv = (real)1 / R_SQRT(ss / (real)D + eps);
        for (int d = 0; d < D; d++)
            o[d] = yr[d] * inv * w[d] * silu(zr[d]);
    }
}

/* ------------------------------------------------------------------------
 * One decode layer of the block, bf16 activations, fp32 state
 *
 * The per-token decode order of [CU]'s header and its glue kernels, with the
 * grouped-query repeat done by index as in [MLX]:
 *   1. widen qkv[n] (bf16) to real; conv1d + SiLU one step over all C
 *      channels, rolling conv_state[n];
 *   2. split the conv output as [q: HK*S | k: HK*S | v: H*S] ([CU]
 *      fc_ssm_qknorm_gqa's input layout);
 *   3. L2-normalise q and k per K-head (eps = l2_eps) and repeat them to
 *      the H V-heads, vh reading K-head vh mod HK;
 *   4. beta = sigmoid(b[n][vh]); g = gate(a[n][vh], dt_bias[vh], A_log[vh]);
 *   5. one recurrence step on state[n] with y = scale * (row . q);
 *   6. out[n][vh] = gated RMSNorm(y[vh], norm_w, widened z[n][vh], eps).
 * Each step calls the stage function above, so the layer is exactly their
 * composition.
 *   qkv [N][C] bf16, z [N][H][S] bf16, a, b [N][H], conv_w [C][K],
 *   A_log, dt_bias [H], norm_w [S], conv_state [N][C][K-1],
 *   state [N][H][S][S], out [N][H][S]
 * ------------------------------------------------------------------------ */
void oracle_decode_block_bf16(const uint16_t *qkv, const uint16_t *z,
                              const real *a, const real *b,
                              const real *conv_w, const real *A_log,
                              const real *dt_bias, const real *norm_w,
                              real *conv_state, real *state, real *out,
                              int n_seqs, int n_k_heads, int n_v_heads, int S,
                              int K, real scale, real l2_eps, real eps)
{
    const int key_dim = n_k_heads * S;
    const int val_dim = n_v_heads * S;
    const int C = 2 * key_dim + val_dim;
    real *x = (real *)malloc(sizeof(real) * (size_t)C);
    real *co = (real *)malloc(sizeof(real) * (size_t)C);
    real *qr = (real *)malloc(sizeof(real) * (size_t)val_dim);
    real *kr = (real *)malloc(sizeof(real) * (size_t)val_dim);
    real *bt = (real *)malloc(sizeof(real) * (size_t)n_v_heads);
    real *gt = (real *)malloc(sizeof(real) * (size_t)n_v_heads);
    real *yt = (real *)malloc(sizeof(real) * (size_t)val_dim);
    real *zt = (real *)malloc(sizeof(real) * (size_t)val_dim);

    for (int n = 0; n < n_seqs; n++) {
        for (int c = 0; c < C; c++)
            x[c] = bf16_to_real(qkv[(size_t)n * C + c]);
        oracle_conv1d_silu_seq(x, conv_w, conv_state + (size_t)n * C * (K - 1),
                               co, 1, 1, C, K);
        oracle_l2norm_gqa(co, qr, 1, n_k_heads, n_v_heads, S, l2_eps);
        oracle_l2norm_gqa(co + key_dim, kr, 1, n_k_heads, n_v_heads, S, l2_eps);
        oracle_sigmoid(b + (size_t)n * n_v_heads, bt, n_v_heads);
        oracle_decay_gate(a + (size_t)n * n_v_heads, dt_bias, A_log, gt,
                          n_v_heads, 1);
        oracle_recurrence_seq(state + (size_t)n * n_v_heads * S * S, qr, kr,
                              co + 2 * key_dim, gt, bt, yt, 1, 1, n_v_heads, S,
                              scale);
        for (int e = 0; e < val_dim; e++)
            zt[e] = bf16_to_real(z[(size_t)n * val_dim + e]);
        oracle_gated_rmsnorm(yt, norm_w, zt, out + (size_t)n * val_dim,
                             n_v_heads, S, eps);
    }
    free(x);
    free(co);
    free(qr);
    free(kr);
    free(bt);
    free(gt);
    free(yt);
    free(zt);
}

/* ------------------------------------------------------------------------
 * Prefill of one layer over T positions, bf16 activations, fp32 state
 *
 * The decode layer above chained over positions, as [CU]'s batched kernels
 * (conv1d_silu_seq, qknorm_gqa_nx with the v pass-through, decay_gate_nx,
 * recurrence_seq) do it; the same stage functions, applied to all T
 * positions of a sequence at once:
 *   qkv [N][T][C] bf16, z [N][T][H][S] bf16, a, b [N][T][H],
 *   conv_state [N][C][K-1], state [N][H][S][S], out [N][T][H][S]
 * ------------------------------------------------------------------------ */
void oracle_prefill_bf16(const uint16_t *qkv, const uint16_t *z, const real *a,
                         const real *b, const real *conv_w, const real *A_log,
                         const real *dt_bias, const real *norm_w,
                         real *conv_state, real *state, real *out, int n_seqs,
                         int n_tokens, int n_k_heads, int n_v_heads, int S,
                         int K, real scale, real l2_eps, real eps)
{
    const int key_dim = n_k_heads * S;
    const int val_dim = n_v_heads * S;
    const int C = 2 * key_dim + val_dim;
    const size_t T = (size_t)n_tokens;
    real *x = (real *)malloc(sizeof(real) * T * C);
    real *co = (real *)malloc(sizeof(real) * T * C);
    real *qs = (real *)malloc(sizeof(real) * T * key_dim);
    real *ks = (real *)malloc(sizeof(real) * T * key_dim);
    real *qr = (real *)malloc(sizeof(real) * T * val_dim);
    real *kr = (real *)malloc(sizeof(real) * T * val_dim);
    real *vv = (real *)malloc(sizeof(real) * T * val_dim);
    real *bt = (real *)malloc(sizeof(real) * T * n_v_heads);
    real *gt = (real *)malloc(sizeof(real) * T * n_v_heads);
    real *yt = (real *)malloc(sizeof(real) * T * val_dim);
    real *zt = (real *)malloc(sizeof(real) * T * val_dim);

    for (int n = 0; n < n_seqs; n++) {
        for (size_t e = 0; e < T * C; e++)
            x[e] = bf16_to_real(qkv[(size_t)n * T * C + e]);
        oracle_conv1d_silu_seq(x, conv_w, conv_state + (size_t)n * C * (K - 1),
                               co, 1, n_tokens, C, K);
        for (size_t t = 0; t < T; t++) {
            for (int e = 0; e < key_dim; e++) {
                qs[t * key_dim + e] = co[t * C + e];
                ks[t * key_dim + e] = co[t * C + key_dim + e];
            }
            for (int e = 0; e < val_dim; e++)
                vv[t * val_dim + e] = co[t * C + 2 * key_dim + e];
        }
        oracle_l2norm_gqa(qs, qr, n_tokens, n_k_heads, n_v_heads, S, l2_eps);
        oracle_l2norm_gqa(ks, kr, n_tokens, n_k_heads, n_v_heads, S, l2_eps);
        oracle_sigmoid(b + (size_t)n * T * n_v_heads, bt, (long)(T * n_v_heads));
        oracle_decay_gate(a + (size_t)n * T * n_v_heads, dt_bias, A_log, gt,
                          n_v_heads, n_tokens);
        oracle_recurrence_seq(state + (size_t)n * n_v_heads * S * S, qr, kr, vv,
                              gt, bt, yt, 1, n_tokens, n_v_heads, S, scale);
        for (size_t e = 0; e < T * val_dim; e++)
            zt[e] = bf16_to_real(z[(size_t)n * T * val_dim + e]);
        oracle_gated_rmsnorm(yt, norm_w, zt, out + (size_t)n * T * val_dim,
                             (long)(T * n_v_heads), S, eps);
    }
    free(x);
    free(co);
    free(qs);
    free(ks);
    free(qr);
    free(kr);
    free(vv);
    free(bt);
    free(gt);
    free(yt);
    free(zt);
}
