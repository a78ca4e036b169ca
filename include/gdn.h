/*
 * gdn.h: C ABI of the Gated DeltaNet (gated delta-rule) SSM block on AMD
 * Instinct MI355X (gfx950).
 *
 * Sources. The operations follow three pages:
 *   [FM]  Foundry, metal/kernels/fm_kernel_ssm.m (host dispatch + MSL kernels)
 *   [CU]  Foundry, cuda_kernels/ssm_gated_delta.cu at commit 775df8ab
 *   [MLX] mlx-native 0.21.1, src/shaders/gated_delta_net_decode.metal
 * Each entry point names the section that defines its operation.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer to memory the caller allocated and
 *     owns. The library never allocates, frees or synchronises; it enqueues
 *     its kernels on `stream` (a hipStream_t; NULL is the default stream)
 *     and returns at once. Faults during execution surface when the caller
 *     synchronises the stream.
 *   - Arrays are dense and row-major (last index fastest), fp32 unless a
 *     parameter says bf16; bf16 values are passed as their 16-bit patterns.
 *   - Arguments are validated before anything is enqueued: on any non-zero
 *     return other than GDN_ELAUNCH nothing was launched and no memory was
 *     touched. GDN_ELAUNCH is the status of the call's own launch (the HIP
 *     runtime's return value for it): an error left pending on the calling
 *     thread by an earlier call is neither reported nor cleared. Of the entry
 *     points that enqueue several kernels (the chunked scan, the prefill), one
 *     that returns GDN_ELAUNCH may have enqueued the kernels before the one
 *     that was rejected. Shape arguments
 *     (heads, state_size, head_dim, conv_dim, conv_kernel) must be positive.
 *     A count argument (n_seqs, n_tokens, rows, n, n_rows) of 0 is an empty
 *     input: the call returns GDN_OK and launches nothing, and its pointers
 *     are not inspected (they may be NULL). A negative count is GDN_ESIZE.
 *   - Shapes are checked before pointers: a call with both a bad shape and a
 *     NULL pointer returns the shape's error code.
 *   - Outputs (y, out, g, ...) must not overlap any input. State arrays are
 *     read and written by the same thread, so they are updated in place.
 *   - Pointers named as float4-accessed must be 16-byte aligned.
 *   - Notation: N = n_seqs, T = n_tokens, H = n_v_heads, HK = n_k_heads,
 *     S = state_size (key dim = value dim = head dim), C = conv_dim,
 *     K = conv_kernel.
 *
 * State layout ([FM] "Delta-rule recurrence", [CU] file header "Config"):
 *   state[n][h][j][i] (N x H x S x S floats) holds entry (i, j) of the
 *   per-head state, i over the key dimension and j over the value dimension:
 *   row j is S contiguous floats over i ("transposed" layout).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define GDN_OK 0
#define GDN_ENULL 1        /* a required pointer is NULL */
#define GDN_ESIZE 2        /* a shape <= 0, a count < 0, too large, or sizes disagree */
#define GDN_EUNSUPPORTED 3 /* a shape the library has no kernel for */
#define GDN_EALIGN 4       /* a float4-accessed pointer is not 16-byte aligned */
#define GDN_ELAUNCH 5      /* the HIP runtime rejected a kernel launch */

/* Text for a return code (static storage, never NULL). */
const char *gdn_strerror(int code);

/* ABI version of this header: 1. */
int gdn_abi_version(void);

/*
 * The gate's per-head factor ssm_a = -exp(A_log) ([CU] fc_ssm_decay_gate,
 * whose comment has it prepared once on the host; [FM] "Decay gate" takes it
 * as its `a` buffer). Every entry point that forms the gate takes ssm_a, as
 * both pages do; a caller that holds the model's A_log prepares ssm_a once
 * per set of parameters with this call.
 *   A_log, ssm_a [n_heads]   (ssm_a may equal A_log: in place)
 * Errors: GDN_ENULL, GDN_ESIZE (n_heads < 0), GDN_ELAUNCH.
 */
int gdn_ssm_a(const float *A_log, float *ssm_a, int n_heads, void *stream);

/*
 * Decay gate ([CU] fc_ssm_decay_gate / fc_ssm_decay_gate_nx; [FM] "Decay
 * gate"):  g[r][h] = ssm_a[h] * softplus(a[r][h] + dt_bias[h]),
 * softplus(u) = u when u > 20, else log1p(exp(u)). With ssm_a = -exp(A_log)
 * <= 0 (gdn_ssm_a), g <= 0, so the decay exp(g) of the recurrence lies in
 * (0, 1].
 *   a, g           [rows][n_heads]
 *   dt_bias, ssm_a [n_heads]
 * Errors: GDN_ENULL, GDN_ESIZE (n_heads <= 0, rows < 0), GDN_ELAUNCH.
 */
int gdn_decay_gate(const float *a, const float *dt_bias, const float *ssm_a, float *g,
                   int n_heads, int64_t rows, void *stream);

/*
 * beta = sigmoid(x) = 1 / (1 + exp(-x)), element-wise ([CU] fc_sigmoid).
 * y may equal x (in place); otherwise they must not overlap.
 *   x, y [n]
 * Errors: GDN_ENULL, GDN_ESIZE (n < 0), GDN_ELAUNCH.
 */
int gdn_sigmoid(const float *x, float *y, int64_t n, void *stream);

/*
 * q/k L2 normalisation with the tiled grouped-query repeat ([CU]
 * fc_ssm_qknorm_gqa / _nx; [MLX] "GQA: tiled mapping"):
 *   xhat = x / max(||x||_2, eps) per K-head; out[r][vh] = xhat[r][vh mod HK].
 *   x   [rows][n_k_heads][head_dim]      (float4-accessed)
 *   out [rows][n_v_heads][head_dim]      (float4-accessed)
 * Errors: GDN_ENULL; GDN_ESIZE (a shape <= 0, rows < 0, n_v_heads not a multiple of
 * n_k_heads); GDN_EUNSUPPORTED (head_dim not a multiple of 4 or > 1024);
 * GDN_EALIGN; GDN_ELAUNCH.
 */
int gdn_l2norm_gqa(const float *x, float *out, int64_t rows, int n_k_heads, int n_v_heads,
                   int head_dim, float eps, void *stream);

/*
 * Causal depthwise conv1d + SiLU, one decode step per sequence ([FM]
 * "Causal depthwise conv1d + SiLU", fmssm_conv1d_silu; [CU] Kernel 2 and
 * fc_ssm_conv1d_silu_slots). Per channel c of sequence n, with
 * hist = conv_state[n][c][0..K-2] (oldest first):
 *   acc = x[n][c] * w[c][K-1] + sum_{u=0..K-2} hist[u] * w[c][u]
 *   out[n][c] = acc / (1 + exp(-acc))
 * then hist drops its oldest entry and appends the raw x[n][c].
 *   x, out     [n_seqs][conv_dim]
 *   w          [conv_dim][conv_kernel]
 *   conv_state [n_seqs][conv_dim][conv_kernel - 1]   (updated in place)
 * Errors: GDN_ENULL, GDN_ESIZE, GDN_EUNSUPPORTED (conv_kernel not in 2..4),
 * GDN_ELAUNCH.
 */
int gdn_conv1d_silu(const float *x, const float *w, float *conv_state, float *out, int n_seqs,
                    int conv_dim, int conv_kernel, void *stream);

/*
 * The same conv over n_tokens positions of each sequence ([FM]
 * fmssm_conv1d_silu_seq; [CU] fc_ssm_conv1d_silu_seq). Every position's
 * output and the final conv_state equal n_tokens single steps bit for bit.
 *   x, out [n_seqs][n_tokens][conv_dim]
 * Any 4-byte alignment is accepted; with conv_dim a multiple of 4, every
 * buffer 16-byte aligned and n_tokens > 8 the scan moves four channels per
 * vector access (same bits, fewer memory instructions).
 * Other arguments and errors as gdn_conv1d_silu.
 */
int gdn_conv1d_silu_seq(const float *x, const float *w, float *conv_state, float *out,
                        int n_seqs, int n_tokens, int conv_dim, int conv_kernel, void *stream);

/*
 * Gated delta-rule recurrence, one token per sequence (decode). [FM]
 * "Delta-rule recurrence" (fmssm_recurrence), [CU] Kernel 1 and
 * fc_ssm_recurrence_slots, [MLX] "Mathematical recurrence". For every
 * (n, h) and every state row j, with r the row and d = exp(g[n][h]):
 *   r = d * r;  pred = r . k;  delta = (v[j] - pred) * beta[n][h];
 *   r = r + k * delta;  y[j] = scale * (r . q)    (read after the update)
 *   state      [n_seqs][n_v_heads][S][S]  (updated in place; float4-accessed)
 *   q, k, v, y [n_seqs][n_v_heads][S]     (q, k after any GQA repeat;
 *                                          q, k float4-accessed)
 *   g, beta    [n_seqs][n_v_heads]        (g <= 0 from gdn_decay_gate)
 * scale multiplies the read-out sum (1/sqrt(S) for the model).
 * Errors: GDN_ENULL, GDN_ESIZE, GDN_EUNSUPPORTED (state_size not in
 * {32, 64, 128, 256}), GDN_EALIGN, GDN_ELAUNCH.
 */
int gdn_recurrence(float *state, const float *q, const float *k, const float *v, const float *g,
                   const float *beta, float *y, int n_seqs, int n_v_heads, int state_size,
                   float scale, void *stream);

/*
 * The recurrence over n_tokens positions of each sequence, the state held
 * on chip between positions and written back once ([FM]
 * fmssm_recurrence_seq; [CU] fc_ssm_recurrence_seq; [MLX] token loop).
 * Every y and the final state equal n_tokens calls of gdn_recurrence bit
 * for bit.
 *   state      [n_seqs][n_v_heads][S][S]            (updated in place)
 *   q, k, v, y [n_seqs][n_tokens][n_v_heads][S]
 *   g, beta    [n_seqs][n_tokens][n_v_heads]
 * Errors as gdn_recurrence.
 */
int gdn_recurrence_seq(float *state, const float *q, const float *k, const float *v,
                       const float *g, const float *beta, float *y, int n_seqs, int n_tokens,
                       int n_v_heads, int state_size, float scale, void *stream);

/* Read-out variants of gdn_recurrence_ex. */
#define GDN_RECUR_EXACT 0 /* y = scale * (updated row . q), as gdn_recurrence */
#define GDN_RECUR_T4 1    /* y = scale * (decayed row . q + delta * (k . q)) */

/*
 * gdn_recurrence with the grouped-query repeat done by index and a choice of
 * read-out. V-head h of sequence n reads K-head h mod n_k_heads of q and k
 * ([MLX] "GQA: tiled mapping"), so q, k are [n_seqs][n_k_heads][S] (pass
 * n_k_heads = n_v_heads for already-repeated q, k). GDN_RECUR_T4 regroups the
 * read-out as [CU]'s "T4" kernel (fc_ssm_recurrence_slots_2pass) does:
 * r_dec . q and r_dec . k are reduced together from the decayed row and
 * y = scale * (r_dec . q + delta * (k . q)). The state is identical to the
 * exact variant bit for bit; y differs from it only by rounding.
 * Errors as gdn_recurrence, plus GDN_ESIZE when n_v_heads is not a multiple
 * of n_k_heads and GDN_EUNSUPPORTED for an unknown variant.
 */
int gdn_recurrence_ex(float *state, const float *q, const float *k, const float *v,
                      const float *g, const float *beta, float *y, int n_seqs, int n_k_heads,
                      int n_v_heads, int state_size, float scale, int variant, void *stream);

/*
 * gdn_recurrence_seq with the grouped-query repeat done by index (q, k are
 * [n_seqs][n_tokens][n_k_heads][S]), optional per-token snapshots for
 * speculative decoding ([CU] fc_ssm_recurrence_seq, "snaps"), and the read-out
 * variant of gdn_recurrence_ex ([CU] "T4", fc_ssm_recurrence_slots_2pass,
 * applied per token). When snaps is not NULL, snaps[n][t] (n_v_heads*S*S
 * floats, the state layout) receives the state after token t of sequence n,
 * so a caller that accepts the first M tokens restores snaps[n][M-1]. snaps
 * [n_seqs][n_tokens][n_v_heads][S][S], 16-byte aligned, caller-owned.
 * variant: GDN_RECUR_EXACT, or GDN_RECUR_T4 (the state, and the snapshots, are
 * those of the exact variant bit for bit; y is reassociated and equals
 * gdn_recurrence_ex with GDN_RECUR_T4 applied token by token, bit for bit).
 * Errors as gdn_recurrence_seq, plus GDN_EUNSUPPORTED for an unknown variant.
 */
int gdn_recurrence_seq_ex(float *state, const float *q, const float *k, const float *v,
                          const float *g, const float *beta, float *y, float *snaps, int n_seqs,
                          int n_tokens, int n_k_heads, int n_v_heads, int state_size, float scale,
                          int variant, void *stream);

/*
 * gdn_conv1d_silu_seq with optional per-position history snapshots ([CU]
 * fc_ssm_conv1d_silu_seq, "snaps"): when snaps is not NULL, snaps[n][t]
 * (conv_dim*(conv_kernel-1) floats, the conv_state layout) receives the
 * history after position t of sequence n.
 *   snaps [n_seqs][n_tokens][conv_dim][conv_kernel - 1], caller-owned.
 * Errors as gdn_conv1d_silu_seq.
 */
int gdn_conv1d_silu_seq_ex(const float *x, const float *w, float *conv_state, float *out,
                           float *snaps, int n_seqs, int n_tokens, int conv_dim, int conv_kernel,
                           void *stream);

/*
 * One decode step from the raw per-token inputs, in one launch: the "glue"
 * of [CU]'s decode path (its q/k L2-norm with the grouped-query repeat,
 * decay-gate and sigmoid kernels) folded into the recurrence:
 *   q^ = q / max(||q||, l2_eps), k^ likewise, per K-head; V-head vh reads
 *   K-head vh mod HK ([MLX] "GQA: tiled mapping");
 *   g = ssm_a[vh] * softplus(a + dt_bias[vh]) (softplus passed through
 *   above 20); beta = 1 / (1 + exp(-b));
 *   then one step of gdn_recurrence with the exact read-out.
 * The result equals gdn_l2norm_gqa (q and k), gdn_decay_gate, gdn_sigmoid
 * and gdn_recurrence_ex chained, bit for bit.
 *   state   [n_seqs][n_v_heads][S][S]   (transposed layout, updated in place)
 *   q, k    [n_seqs][n_k_heads][S]      raw (not normalised), per K-head
 *   v, y    [n_seqs][n_v_heads][S]
 *   a, b    [n_seqs][n_v_heads]         gate and beta inputs
 *   ssm_a, dt_bias [n_v_heads]
 * Errors: GDN_ENULL; GDN_ESIZE (a size <= 0, n_seqs < 0, n_v_heads not a
 * multiple of n_k_heads); GDN_EUNSUPPORTED (S not in {32, 64, 128, 256});
 * GDN_EALIGN (state, q or k not 16-byte aligned); GDN_ELAUNCH.
 */
int gdn_decode_step(float *state, const float *q, const float *k, const float *v,
                    const float *a, const float *b, const float *ssm_a, const float *dt_bias,
                    float *y, int n_seqs, int n_k_heads, int n_v_heads, int state_size,
                    float scale, float l2_eps, void *stream);

/*
 * Gated RMSNorm ([FM] "Gated RMSNorm"; [CU] Kernel 3): per row of head_dim
 * values, out = y / sqrt(mean(y^2) + eps) * w * silu(z), silu(z) =
 * z / (1 + exp(-z)). The weight is shared by every row (every head).
 *   y, z, out [n_rows][head_dim]   w [head_dim]   (all float4-accessed)
 * Errors: GDN_ENULL, GDN_ESIZE, GDN_EUNSUPPORTED (head_dim not a multiple
 * of 4 or > 1024), GDN_EALIGN, GDN_ELAUNCH.
 */
int gdn_gated_rmsnorm(const float *y, const float *w, const float *z, float *out,
                      int64_t n_rows, int head_dim, float eps, void *stream);

/*
 * One decode layer of the block, fused into one kernel: bf16 activations,
 * fp32 state. The per-token order of [CU]'s decode path (its file header and
 * "glue" kernels) with the grouped-query repeat done by index ([MLX]):
 *   1. conv1d + SiLU one step on the widened qkv[n] (all C channels),
 *      rolling conv_state[n];
 *   2. split the conv output as [q: HK*S | k: HK*S | v: H*S];
 *   3. L2-normalise q and k per K-head (l2_eps); V-head vh reads K-head
 *      vh mod HK;
 *   4. beta = sigmoid(b[n][vh]); g = ssm_a[vh] *
 *      softplus(a[n][vh] + dt_bias[vh]), ssm_a = -exp(A_log) (gdn_ssm_a);
 *   5. one recurrence step of state[n][vh], y = scale * (row . q);
 *   6. out[n][vh] = gated RMSNorm(y[vh], norm_w, widened z[n][vh], eps).
 *   qkv        [n_seqs][C] bf16, C = 2*HK*S + H*S
 *   z          [n_seqs][n_v_heads][S] bf16
 *   a, b       [n_seqs][n_v_heads]
 *   conv_w     [C][conv_kernel];  ssm_a, dt_bias [n_v_heads];  norm_w [S]
 *   conv_state [n_seqs][C][conv_kernel - 1]   (updated in place)
 *   state      [n_seqs][n_v_heads][S][S]      (updated in place)
 *   out        [n_seqs][n_v_heads][S]
 * Errors: GDN_ENULL; GDN_ESIZE (a size <= 0 or H not a multiple of HK);
 * GDN_EUNSUPPORTED (S != 128, H/HK > 4, conv_kernel not in 2..4);
 * GDN_EALIGN (state, norm_w or out not 16-byte aligned); GDN_ELAUNCH.
 */
int gdn_decode_block_bf16(const uint16_t *qkv, const uint16_t *z, const float *a,
                          const float *b, const float *conv_w, const float *ssm_a,
                          const float *dt_bias, const float *norm_w, float *conv_state,
                          float *state, float *out, int n_seqs, int n_k_heads, int n_v_heads,
                          int state_size, int conv_kernel, float scale, float l2_eps, float eps,
                          void *stream);

/*
 * Workspace, in bytes, that gdn_decode_block_bf16_ex needs (0 for invalid
 * sizes): one 32-bit counter per (sequence, K-head) and per (sequence,
 * V-head).
 */
size_t gdn_decode_block_workspace_bytes(int n_seqs, int n_k_heads, int n_v_heads);

/*
 * The decode layer of gdn_decode_block_bf16 (same steps, same arguments,
 * same results bit for bit), with the state of each V-head split over
 * workgroups of 64 rows instead of one workgroup per K-head: faster when
 * the state streams from HBM. Each workgroup convolves and normalises the
 * q and k of its K-head itself; the last workgroup of a K-head to read
 * their history rolls it, and the last workgroup of a V-head applies the
 * gated norm, both found through counters in the workspace.
 *   workspace  caller-owned device memory of at least
 *              gdn_decode_block_workspace_bytes(...) bytes, 4-byte aligned,
 *              ZERO before the first call; every completed call leaves it
 *              zero again. Calls that may run at the same time (on
 *              different streams) need workspaces of their own. A workspace
 *              that is not zero when a call starts (one shared by calls that
 *              overlap, or left by a launch that did not complete) gives
 *              wrong outputs without an error and is not cleared by later
 *              calls: zero it again (hipMemset) before reusing it.
 *   other arguments as gdn_decode_block_bf16.
 * Errors: as gdn_decode_block_bf16; also GDN_ENULL (workspace NULL),
 * GDN_ESIZE (workspace too small), GDN_EALIGN (workspace not 4-byte aligned).
 */
int gdn_decode_block_bf16_ex(const uint16_t *qkv, const uint16_t *z, const float *a,
                             const float *b, const float *conv_w, const float *ssm_a,
                             const float *dt_bias, const float *norm_w, float *conv_state,
                             float *state, float *out, void *workspace, size_t workspace_bytes,
                             int n_seqs, int n_k_heads, int n_v_heads, int state_size,
                             int conv_kernel, float scale, float l2_eps, float eps, void *stream);

/* Capacity of the library-owned counter array of gdn_decode_block_bf16_noalloc,
   per GPU: n_seqs * (n_k_heads + n_v_heads) may not exceed it. */
#define GDN_NOALLOC_MAX_COUNTERS 65536

/*
 * gdn_decode_block_bf16_ex without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same steps, arguments (but the
 * workspace) and results, bit for bit. Its counters live in a library-owned
 * device array of GDN_NOALLOC_MAX_COUNTERS 32-bit counters (256 KiB) on each
 * GPU it runs on, held until the process ends; the call itself allocates
 * nothing. The array starts zero and every completed call leaves it zero.
 * Calls that overlap on one GPU (on different streams, or from several host
 * threads) share the array and race: the caller serialises them, or uses
 * gdn_decode_block_bf16_ex with a workspace of its own per stream.
 * Errors: as gdn_decode_block_bf16; GDN_ESIZE also when n_seqs * (n_k_heads +
 * n_v_heads) > GDN_NOALLOC_MAX_COUNTERS; GDN_ELAUNCH also when the array's
 * device address cannot be found (no usable GPU).
 */
int gdn_decode_block_bf16_noalloc(const uint16_t *qkv, const uint16_t *z, const float *a,
                                  const float *b, const float *conv_w, const float *ssm_a,
                                  const float *dt_bias, const float *norm_w, float *conv_state,
                                  float *state, float *out, int n_seqs, int n_k_heads,
                                  int n_v_heads, int state_size, int conv_kernel, float scale,
                                  float l2_eps, float eps, void *stream);

/*
 * Workspace, in bytes, that gdn_prefill_bf16 and gdn_prefill_bf16_ex (either
 * scan) need for these sizes (0 for invalid sizes): normalised q and k per
 * K-head, v, g, beta and y, fp32, and the chunked scan's workspace.
 */
size_t gdn_prefill_workspace_bytes(int n_seqs, int n_tokens, int n_k_heads, int n_v_heads,
                                   int state_size);

/*
 * Prefill of one layer over n_tokens positions, bf16 activations, fp32 state:
 * the decode layer of gdn_decode_block_bf16 chained over positions ([CU]'s
 * batched "_nx" / "_seq" kernels: conv1d_silu_seq, qknorm_gqa_nx with the v
 * pass-through, decay_gate_nx, recurrence_seq; then the gated norm).
 *   1. conv1d + SiLU over the positions of the widened qkv (rolls
 *      conv_state), split [q | k | v], q and k L2-normalised per K-head
 *      (l2_eps), g = ssm_a*softplus(a + dt_bias), beta = sigmoid(b);
 *   2. the sequential scan, V-head vh reading K-head vh mod HK, y = scale *
 *      (row . q);
 *   3. out = gated RMSNorm(y, norm_w, widened z, eps).
 * The result equals n_tokens calls of gdn_decode_block_bf16 bit for bit.
 *   qkv        [n_seqs][n_tokens][C] bf16, C = 2*HK*S + H*S (8-byte aligned)
 *   z          [n_seqs][n_tokens][n_v_heads][S] bf16 (8-byte aligned)
 *   a, b       [n_seqs][n_tokens][n_v_heads]
 *   conv_w [C][conv_kernel]; ssm_a, dt_bias [n_v_heads]; norm_w [S]
 *   conv_state [n_seqs][C][conv_kernel-1], state [n_seqs][n_v_heads][S][S]
 *              (both updated in place)
 *   out        [n_seqs][n_tokens][n_v_heads][S]
 *   workspace  caller-owned device memory of at least
 *              gdn_prefill_workspace_bytes(...) bytes, 256-byte aligned; its
 *              contents on return are unspecified
 * Errors: GDN_ENULL; GDN_ESIZE (a shape <= 0, a count < 0, H not a multiple
 * of HK, workspace too small); GDN_EUNSUPPORTED (S != 128, conv_kernel not in
 * 2..4); GDN_EALIGN; GDN_ELAUNCH.
 */
int gdn_prefill_bf16(const uint16_t *qkv, const uint16_t *z, const float *a, const float *b,
                     const float *conv_w, const float *ssm_a, const float *dt_bias,
                     const float *norm_w, float *conv_state, float *state, float *out,
                     void *workspace, size_t workspace_bytes, int n_seqs, int n_tokens,
                     int n_k_heads, int n_v_heads, int state_size, int conv_kernel, float scale,
                     float l2_eps, float eps, void *stream);

/*
 * Workspace, in bytes, that gdn_recurrence_seq_chunked needs (0 for invalid
 * sizes or an unsupported state size): per (sequence, V-head, 64-position
 * chunk) 8448 floats (per-position decay factors and beta, and two 64 x 64
 * matrices).
 */
size_t gdn_chunked_workspace_bytes(int n_seqs, int n_tokens, int n_v_heads, int state_size);

/*
 * The scan of gdn_recurrence_seq_ex (no snapshots) in chunked form: the
 * positions are taken 64 at a time and the delta rule over a chunk is applied
 * as matrix products (WY-style blocking, fp32 MFMA): a preparation kernel
 * builds each chunk's (I + A)^-1 and masked Q K^T for all chunks in parallel,
 * then a scan kernel carries the state through the chunks in order. The pages name a chunked
 * prefill and keep the sequential scan as its reference ([FM] "softplus"
 * comment and the sequential-scan section) without giving its algorithm.
 * Same arguments and layouts as gdn_recurrence_seq_ex, plus a caller-owned
 * workspace of at least gdn_chunked_workspace_bytes(...) bytes (16-byte
 * aligned; contents on return unspecified). y and the state agree with the
 * sequential scan within the fp32 tolerance, not bit for bit.
 * Errors: GDN_ENULL; GDN_ESIZE (as gdn_recurrence_seq_ex, or workspace too
 * small); GDN_EUNSUPPORTED (state_size != 128); GDN_EALIGN (state, q, k, v, y
 * or workspace not 16-byte aligned); GDN_ELAUNCH.
 */
int gdn_recurrence_seq_chunked(float *state, const float *q, const float *k, const float *v,
                               const float *g, const float *beta, float *y, void *workspace,
                               size_t workspace_bytes, int n_seqs, int n_tokens, int n_k_heads,
                               int n_v_heads, int state_size, float scale, void *stream);

#define GDN_SCAN_SEQUENTIAL 0 /* the scan of gdn_recurrence_seq_ex */
#define GDN_SCAN_CHUNKED 1    /* the scan of gdn_recurrence_seq_chunked */

/*
 * gdn_prefill_bf16 with a choice of scan for stage 2. GDN_SCAN_SEQUENTIAL is
 * gdn_prefill_bf16 itself (equal to chained gdn_decode_block_bf16 calls bit
 * for bit); GDN_SCAN_CHUNKED runs the chunked form of the same scan, which
 * agrees with it within the fp32 tolerance. Same arguments, layouts and
 * workspace as gdn_prefill_bf16.
 * Errors: as gdn_prefill_bf16, and GDN_EUNSUPPORTED for an unknown scan.
 */
int gdn_prefill_bf16_ex(const uint16_t *qkv, const uint16_t *z, const float *a, const float *b,
                        const float *conv_w, const float *ssm_a, const float *dt_bias,
                        const float *norm_w, float *conv_state, float *state, float *out,
                        void *workspace, size_t workspace_bytes, int n_seqs, int n_tokens,
                        int n_k_heads, int n_v_heads, int state_size, int conv_kernel, float scale,
                        float l2_eps, float eps, int scan, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
