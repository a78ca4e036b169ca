/*
 * A plain C caller of the library, built by tests/test_abi_cpu.py as strict
 * C11 and as C++17 against include/gdn.h and linked
 * with libgdn.so. Every entry point is called once or more on an argument
 * path that returns before anything is launched (no GPU is needed), through
 * the header's own prototypes, and the return code is checked. A header that
 * does not compile as C, a declared function the library does not export, or
 * a prototype that disagrees with the library's argument order shows up here
 * as a build error, a link error or a wrong code. No call here may pass
 * validation: the buffers are host memory, which no kernel may be given.
 */
#include <stdint.h>
#include <stdio.h>

#include "gdn.h"

static int failures = 0;

static void expect(const char *what, long got, long want) {
  if (got != want) {
    printf("FAIL %s: got %ld, want %ld\n", what, got, want);
    ++failures;
  }
}

#define EXPECT(call, want) expect(#call, (long)(call), (long)(want))

/* Host buffers: valid addresses that the checks may inspect for alignment
   but never dereference. */
static float buf[256] __attribute__((aligned(256)));
static uint16_t buf16[256] __attribute__((aligned(256)));

int main(void) {
  float *f = buf;
  const float *cf = buf;
  float *mis = buf + 1; /* 4-byte aligned only */

  EXPECT(gdn_abi_version(), 1);
  EXPECT(gdn_strerror(GDN_OK) != NULL, 1);
  EXPECT(gdn_strerror(12345) != NULL, 1);

  EXPECT(gdn_decay_gate(NULL, cf, cf, f, 4, 1, NULL), GDN_ENULL);
  EXPECT(gdn_decay_gate(cf, cf, cf, f, 0, 1, NULL), GDN_ESIZE);
  EXPECT(gdn_decay_gate(NULL, NULL, NULL, NULL, 4, 0, NULL), GDN_OK);

  EXPECT(gdn_sigmoid(NULL, f, 3, NULL), GDN_ENULL);
  EXPECT(gdn_sigmoid(cf, f, -1, NULL), GDN_ESIZE);
  EXPECT(gdn_sigmoid(NULL, NULL, 0, NULL), GDN_OK);

  EXPECT(gdn_l2norm_gqa(NULL, f, 1, 2, 4, 32, 1e-6f, NULL), GDN_ENULL);
  EXPECT(gdn_l2norm_gqa(cf, f, 1, 2, 3, 32, 1e-6f, NULL), GDN_ESIZE);

  EXPECT(gdn_conv1d_silu(NULL, cf, f, f, 1, 8, 4, NULL), GDN_ENULL);
  EXPECT(gdn_conv1d_silu(cf, cf, f, f, 1, 8, 5, NULL), GDN_EUNSUPPORTED);
  EXPECT(gdn_conv1d_silu(NULL, NULL, NULL, NULL, 0, 8, 4, NULL), GDN_OK);
  EXPECT(gdn_conv1d_silu_seq(cf, cf, f, f, 1, -1, 8, 4, NULL), GDN_ESIZE);
  EXPECT(gdn_conv1d_silu_seq(NULL, NULL, NULL, NULL, 1, 0, 8, 4, NULL), GDN_OK);
  EXPECT(gdn_conv1d_silu_seq_ex(cf, cf, f, f, NULL, 1, 1, 8, 5, NULL), GDN_EUNSUPPORTED);

  EXPECT(gdn_recurrence(NULL, cf, cf, cf, cf, cf, f, 1, 2, 32, 1.0f, NULL), GDN_ENULL);
  EXPECT(gdn_recurrence(f, cf, cf, cf, cf, cf, f, 1, 2, 48, 1.0f, NULL), GDN_EUNSUPPORTED);
  EXPECT(gdn_recurrence(mis, cf, cf, cf, cf, cf, f, 1, 2, 32, 1.0f, NULL), GDN_EALIGN);
  EXPECT(gdn_recurrence_seq(f, cf, cf, cf, cf, cf, f, 1, 0, 2, 32, 1.0f, NULL), GDN_OK);
  EXPECT(gdn_recurrence_seq(f, cf, cf, cf, cf, cf, f, 1, -2, 2, 32, 1.0f, NULL), GDN_ESIZE);
  EXPECT(gdn_recurrence_ex(f, cf, cf, cf, cf, cf, f, 1, 2, 4, 32, 1.0f, 7, NULL),
         GDN_EUNSUPPORTED);
  EXPECT(gdn_recurrence_ex(f, cf, cf, cf, cf, cf, f, 1, 3, 4, 32, 1.0f, GDN_RECUR_T4, NULL),
         GDN_ESIZE);
  EXPECT(gdn_recurrence_seq_ex(f, cf, cf, cf, cf, cf, f, NULL, 1, 3, 2, 4, 32, 1.0f, 7, NULL),
         GDN_EUNSUPPORTED);
  EXPECT(gdn_recurrence_seq_ex(f, cf, cf, cf, cf, cf, f, mis, 1, 3, 2, 4, 32, 1.0f,
                               GDN_RECUR_EXACT, NULL),
         GDN_EALIGN);
  EXPECT(gdn_recurrence_seq_ex(f, cf, cf, cf, cf, cf, f, NULL, 1, 0, 2, 4, 32, 1.0f,
                               GDN_RECUR_T4, NULL),
         GDN_OK);

  EXPECT(gdn_decode_step(f, cf, cf, cf, NULL, cf, cf, cf, f, 1, 16, 32, 128, 0.1f, 1e-6f, NULL),
         GDN_ENULL);
  EXPECT(gdn_decode_step(f, cf, cf, cf, cf, cf, cf, cf, f, 1, 16, 32, 96, 0.1f, 1e-6f, NULL),
         GDN_EUNSUPPORTED);

  EXPECT(gdn_gated_rmsnorm(NULL, cf, cf, f, 1, 32, 1e-6f, NULL), GDN_ENULL);
  EXPECT(gdn_gated_rmsnorm(cf, cf, cf, f, 1, 0, 1e-6f, NULL), GDN_ESIZE);

  EXPECT(gdn_decode_block_bf16(NULL, buf16, cf, cf, cf, cf, cf, cf, f, f, f, 1, 16, 32, 128, 4,
                               0.1f, 1e-6f, 1e-6f, NULL),
         GDN_ENULL);
  EXPECT(gdn_decode_block_bf16(buf16, buf16, cf, cf, cf, cf, cf, cf, f, f, f, 1, 16, 32, 64, 4,
                               0.1f, 1e-6f, 1e-6f, NULL),
         GDN_EUNSUPPORTED);

  /* one counter per (sequence, K-head) and per (sequence, V-head) */
  EXPECT(gdn_decode_block_workspace_bytes(2, 16, 32), (2L * 16 + 2L * 32) * 4);
  EXPECT(gdn_decode_block_workspace_bytes(2, 16, 24), 0);
  EXPECT(gdn_decode_block_bf16_ex(buf16, buf16, cf, cf, cf, cf, cf, cf, f, f, f, f, 16, 1, 16, 32,
                                  128, 4, 0.1f, 1e-6f, 1e-6f, NULL),
         GDN_ESIZE); /* workspace too small */
  EXPECT(gdn_decode_block_bf16_ex(buf16, buf16, cf, cf, cf, cf, cf, cf, f, f, f, NULL, 4096, 1,
                                  16, 32, 128, 4, 0.1f, 1e-6f, 1e-6f, NULL),
         GDN_ENULL);

  EXPECT(gdn_prefill_workspace_bytes(1, 64, 16, 32, 128) > 0, 1);
  EXPECT(gdn_prefill_workspace_bytes(1, 64, 0, 32, 128), 0);
  EXPECT(gdn_prefill_bf16(buf16, buf16, cf, cf, cf, cf, cf, cf, f, f, f, f, 16, 1, 64, 16, 32,
                          128, 4, 0.1f, 1e-6f, 1e-6f, NULL),
         GDN_ESIZE); /* workspace too small */
  EXPECT(gdn_prefill_bf16_ex(buf16, buf16, cf, cf, cf, cf, cf, cf, f, f, f, f, 16, 1, 64, 16, 32,
                             128, 4, 0.1f, 1e-6f, 1e-6f, 9, NULL),
         GDN_EUNSUPPORTED);

  /* one 64-position chunk of 4 heads: 8448 floats per head */
  EXPECT(gdn_chunked_workspace_bytes(1, 64, 4, 128), 4L * 8448 * 4);
  EXPECT(gdn_chunked_workspace_bytes(1, 64, 4, 64), 0);
  EXPECT(gdn_recurrence_seq_chunked(f, cf, cf, cf, cf, cf, f, f, 16, 1, 64, 4, 4, 128, 1.0f,
                                    NULL),
         GDN_ESIZE); /* workspace too small */
  EXPECT(gdn_recurrence_seq_chunked(f, cf, cf, cf, cf, cf, f, f, 1 << 20, 1, 64, 4, 4, 64, 1.0f,
                                    NULL),
         GDN_EUNSUPPORTED);

  EXPECT(gdn_decode_block_bf16_noalloc(buf16, buf16, cf, cf, cf, cf, cf, cf, f, f, f, 1366, 16, 32,
                                       128, 4, 0.1f, 1e-6f, 1e-6f, NULL),
         GDN_ESIZE); /* 1366 * 48 counters > GDN_NOALLOC_MAX_COUNTERS */
  EXPECT(gdn_decode_block_bf16_noalloc(NULL, buf16, cf, cf, cf, cf, cf, cf, f, f, f, 3, 16, 32,
                                       128, 4, 0.1f, 1e-6f, 1e-6f, NULL),
         GDN_ENULL);
  EXPECT(gdn_ssm_a(NULL, f, 4, NULL), GDN_ENULL);
  EXPECT(gdn_ssm_a(cf, NULL, 4, NULL), GDN_ENULL);
  EXPECT(gdn_ssm_a(cf, f, -1, NULL), GDN_ESIZE);
  EXPECT(gdn_ssm_a(NULL, NULL, 0, NULL), GDN_OK);

  printf("%d failures\n", failures);
  return failures != 0;
}
