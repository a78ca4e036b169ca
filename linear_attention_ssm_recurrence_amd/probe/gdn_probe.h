/*
 * gdn_probe.h: measurement probes for the benchmark, built as their own
 * library (libgdn_probe.so) beside libgdn.so and not part of the library's
 * interface.
 *
 * They are not steps of the Gated DeltaNet block. The benchmark calls them to
 * measure what this particular MI355X achieves, so that a kernel's roofline
 * fraction can be stated against the measured figure as well as against the
 * published peak.
 */
#ifndef GDN_PROBE_H
#define GDN_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fp32 FMA issue rate: n_blocks workgroups of 256 threads, each thread
 * running 16 independent chains of `iters` dependent v_fma_f32 (unpacked, as
 * every kernel of libgdn.so is built), 2 flop each. Total work
 * n_blocks * 256 * iters * 32 flop. Each thread writes the sum of its chains
 * to out[block * 256 + thread] (n_blocks * 256 floats of caller-owned device
 * memory), so nothing is optimised away; the values carry no meaning. The
 * kernel is enqueued on `stream` (a hipStream_t).
 * Returns 0 when the kernel was enqueued; 1 for a NULL out; 2 for n_blocks or
 * iters <= 0 or n_blocks > 2^20 (nothing launched); 5 when the runtime
 * rejected the launch.
 */
int gdn_probe_fma(float *out, int n_blocks, int iters, float a, float b, void *stream);

/*
 * Matrix-instruction issue rate: n_blocks workgroups of 256 threads (four
 * waves), each wave running `chains` independent accumulator chains of
 * `iters` dependent matrix instructions: kind 0 v_mfma_f32_16x16x4f32 (2048
 * flop each), kind 1 v_mfma_f32_16x16x32_bf16 (16384 flop each). With
 * n_blocks = 256 there is one wave per SIMD. out as gdn_probe_fma.
 * Returns 0, 1 (NULL out), 2 (bad n_blocks or iters), 3 (bad kind or chains
 * not 1, 2 or 4), or 5 (launch rejected).
 */
int gdn_probe_mfma(int kind, int chains, float *out, int n_blocks, int iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PROBE_H */
