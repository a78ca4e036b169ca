/*
 * gdn_probe.h: measurement probes exported by libgdn.so.
 *
 * These are not steps of the Gated DeltaNet block. A benchmark calls them to
 * measure what this particular MI355X achieves, so that a kernel's roofline
 * fraction can be stated against the measured figure as well as against the
 * published peak. Same conventions as gdn.h: device pointers owned by the
 * caller, asynchronous on `stream`, validated before anything is launched,
 * return codes from gdn.h.
 */
#ifndef GDN_PROBE_H
#define GDN_PROBE_H

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fp32 FMA issue rate: n_blocks workgroups of 256 threads, each thread
 * running 16 independent chains of `iters` dependent v_fma_f32 (unpacked, as
 * every kernel of this library is built), 2 flop each. Total work
 * n_blocks * 256 * iters * 32 flop. Each thread writes the sum of its chains
 * to out[block * 256 + thread] (n_blocks * 256 floats), so nothing is
 * optimised away; the values carry no meaning.
 * Errors: GDN_ESIZE (n_blocks or iters <= 0, or n_blocks > 2^20); GDN_ENULL;
 * GDN_ELAUNCH.
 */
int gdn_probe_fma(float *out, int n_blocks, int iters, float a, float b, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PROBE_H */
