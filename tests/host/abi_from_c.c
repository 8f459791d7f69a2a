/*
 * abi_from_c.c - a C99 consumer of include/fa.h (host only, no GPU needed).
 *
 * Compiled with the host C compiler against the header and linked with
 * libfa_mi355x.so, it calls every entry point with arguments that the library must
 * reject before any HIP call (the pointers are never dereferenced), and checks the
 * error code of each.  It covers the argument rules stated in fa.h: NULL pointers,
 * sizes, windows, dtype, alignment, head grouping, and grids whose work-item count
 * would not fit in 32 bits.  Prints "ok <n>" and exits 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int n_checks = 0, n_failed = 0;

static void expect(int got, int want, const char* what, int line) {
  ++n_checks;
  if (got != want) {
    ++n_failed;
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

int main(void) {
  /* fake, 16-byte aligned device addresses: every call below fails validation first */
  void* P = (void*)(uintptr_t)0x100000;
  float* F = (float*)(uintptr_t)0x200000;
  const int* I = (const int*)(uintptr_t)0x300000;
  void* odd = (void*)(uintptr_t)0x100008;
  hipStream_t s = 0;

  /* status strings */
  EXPECT(strcmp(fa_status_str(FA_OK), "FA_OK"), 0);
  EXPECT(fa_status_str(FA_ERR_INVALID_ARG) != NULL && strstr(fa_status_str(FA_ERR_INVALID_ARG), "INVALID") != NULL, 1);
  EXPECT(strcmp(fa_status_str(42), "unknown status"), 0);

  /* fa_fwd */
  EXPECT(fa_fwd(NULL, P, P, P, F, 1, 4, 4, 2, 64, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, NULL, F, 1, 4, 4, 2, 64, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, NULL, 1, 4, 4, 2, 64, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, F, 0, 4, 4, 2, 64, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 4, 2, 64, 0.125f, 0, -2, -1, NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 4, 2, 64, (float)INFINITY, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 4, 2, 64, (float)NAN, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 4, 2, 96, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 4, 2, 64, 0.125f, 0, -1, -1, NULL, 0, 2, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 4, 2, 64, 0.125f, 0, -1, -1, F, 2, FA_FP16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(odd, P, P, P, F, 1, 4, 4, 2, 64, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, F, 1, (1 << 30) + 1, 4, 2, 64, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd(P, P, P, P, F, 1, 4, 4, 1 << 16, 128, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s), FA_ERR_UNSUPPORTED);
  /* grids: 2^24 four-wave workgroups of 256 threads (2^32 work-items) */
  EXPECT(fa_fwd(P, P, P, P, F, 1 << 17, 128, 128, 128, 64, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);
  /* 2^23 eight-wave workgroups of 512 threads (headdim 128, unmasked, 4096 query rows) */
  EXPECT(fa_fwd(P, P, P, P, F, 1 << 11, 4096, 4096, 256, 128, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);

  /* fa_fwd_splitkv */
  EXPECT(fa_fwd_splitkv(P, P, P, F, F, 1, 1, 4, 2, 64, 0.125f, 1, -1, -1, NULL, 0, FA_BF16, 0, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_splitkv(P, P, P, F, F, 1, 1, 4, 2, 64, 0.125f, 1, -1, -1, NULL, 0, FA_BF16, 5, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_splitkv(P, P, P, NULL, F, 1, 1, 4, 2, 64, 0.125f, 1, -1, -1, NULL, 0, FA_BF16, 2, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_splitkv(P, P, P, (float*)odd, F, 1, 1, 4, 2, 64, 0.125f, 1, -1, -1, NULL, 0, FA_BF16, 2, s),
         FA_ERR_INVALID_ARG);
  /* 2^24 vector-ALU decode workgroups: batch 2^16 x 16 heads x 16 splits */
  EXPECT(fa_fwd_splitkv(P, P, P, F, F, 1 << 16, 1, 64, 16, 64, 0.125f, 1, -1, -1, NULL, 0, FA_BF16, 16, s),
         FA_ERR_INVALID_ARG);

  /* fa_fwd_varlen */
  EXPECT(fa_fwd_varlen(P, P, P, P, F, NULL, I, 2, 8, 8, 10, 4, 2, 128, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_varlen(P, P, P, P, F, I, I, 2, 8, 8, 10, 4, 3, 128, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_varlen(P, P, P, P, F, I, I, 2, 8, 8, 0, 4, 2, 128, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_varlen(P, P, P, P, F, I, I, 2, 8, 8, 10, 4, 2, 80, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_UNSUPPORTED);

  /* fa_combine */
  EXPECT(fa_combine(NULL, F, P, F, 1, 1, 1, 64, 2, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_combine(F, F, P, F, 1, 1, 1, 64, 0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_combine(F, F, P, F, 1, 1, 1, 100, 2, FA_BF16, s), FA_ERR_UNSUPPORTED);
  EXPECT(fa_combine(F, F, P, F, 1, 1, 1, 64, 2, 9, s), FA_ERR_INVALID_ARG);
  /* one workgroup per row: 2^24 rows is one past the grid limit */
  EXPECT(fa_combine(F, F, P, F, 1, 1 << 24, 1, 64, 2, FA_BF16, s), FA_ERR_INVALID_ARG);

  /* fa_fwd_kvcache */
  EXPECT(fa_fwd_kvcache(P, P, P, NULL, I, 256, 4, NULL, NULL, 0, NULL, NULL, 0, P, F, F, F, 16, 2, 1, 8, 2, 128,
                        0.1f, 1, -1, -1, NULL, 0, FA_BF16, 0, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_kvcache(P, P, P, I, I, 100, 4, NULL, NULL, 0, NULL, NULL, 0, P, F, F, F, 16, 2, 1, 8, 2, 128,
                        0.1f, 1, -1, -1, NULL, 0, FA_BF16, 0, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_kvcache(P, P, P, I, I, 256, 4, NULL, NULL, 0, NULL, NULL, 0, P, F, F, F, 16, 2, 9, 8, 2, 128,
                        0.1f, 1, -1, -1, NULL, 0, FA_BF16, 0, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_kvcache(P, P, P, I, I, 256, 4, NULL, NULL, 0, F, NULL, 0, P, F, F, F, 16, 2, 1, 8, 2, 128,
                        0.1f, 1, -1, -1, NULL, 0, FA_BF16, 0, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_kvcache(P, P, P, I, I, 256, 4, NULL, NULL, 0, NULL, NULL, 0, P, F, F, F, 16, 2, 1, 8, 2, 128,
                        0.1f, 1, -1, -1, NULL, 0, FA_BF16, 17, s), FA_ERR_INVALID_ARG);
  /* more appended rows than the cache holds */
  EXPECT(fa_fwd_kvcache(P, P, P, I, NULL, 4, 1, P, P, 5, NULL, NULL, 0, P, F, F, F, 16, 2, 1, 8, 2, 128,
                        0.1f, 1, -1, -1, NULL, 0, FA_BF16, 1, s), FA_ERR_INVALID_ARG);
  /* the combine grid: batch 2^21 x 8 heads = 2^24 rows */
  EXPECT(fa_fwd_kvcache(P, P, P, I, NULL, 256, 1, NULL, NULL, 0, NULL, NULL, 0, P, F, F, F, 16, 1 << 21, 1, 8, 8,
                        64, 0.1f, 1, -1, -1, NULL, 0, FA_BF16, 1, s), FA_ERR_INVALID_ARG);

  /* fa_fwd_kvcache_noalloc: 2032 splits of batch 2 x 8 heads x headdim 128 fit its buffer */
  EXPECT(fa_fwd_kvcache_noalloc(P, P, P, NULL, I, 256, 4, NULL, NULL, 0, NULL, NULL, 0, P, F, 2, 1, 8, 2, 128, 0.1f,
                                1, -1, -1, NULL, 0, FA_BF16, 0, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_kvcache_noalloc(P, P, P, I, I, 256, 4, NULL, NULL, 0, NULL, NULL, 0, P, F, 2, 1, 8, 2, 128, 0.1f,
                                1, -1, -1, NULL, 0, FA_BF16, 2033, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_fwd_kvcache_noalloc(P, P, P, I, I, 256, 4, NULL, NULL, 0, NULL, NULL, 0, P, F, 1 << 20, 1, 8, 2, 128,
                                0.1f, 1, -1, -1, NULL, 0, FA_BF16, 1, s), FA_ERR_INVALID_ARG);

  /* fa_bwd */
  EXPECT(fa_bwd(P, P, P, P, F, P, P, P, P, NULL, 1, 4, 4, 2, 128, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_bwd(P, P, P, P, F, P, odd, P, P, F, 1, 4, 4, 2, 128, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);
  EXPECT(fa_bwd(P, P, P, P, F, P, P, P, P, F, 1, 4, 4, 2, 32, 0.125f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_UNSUPPORTED);
  /* the dQ grid: 2^23 (batch, head) pairs of two 128-row query tiles make 2^24 workgroups */
  EXPECT(fa_bwd(P, P, P, P, F, P, P, P, P, F, 1 << 23, 256, 128, 1, 256, 0.0625f, 0, -1, -1, NULL, 0, FA_BF16, s),
         FA_ERR_INVALID_ARG);

  /* fa_bwd_varlen */
  EXPECT(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, F, I, NULL, 2, 8, 8, 10, 12, 4, 2, 128, 0.125f, 0, -1, -1, NULL,
                       0, FA_BF16, s), FA_ERR_INVALID_ARG);
  EXPECT(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, F, I, I, 2, 8, 8, 10, 0, 4, 2, 128, 0.125f, 0, -1, -1, NULL,
                       0, FA_BF16, s), FA_ERR_INVALID_ARG);
  /* the dQ grid: 2^23 sequences of up to two 128-row query tiles make 2^24 workgroups */
  EXPECT(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, F, I, I, 1 << 23, 256, 8, 12, 12, 1, 1, 256, 0.0625f, 0, -1, -1,
                       NULL, 0, FA_BF16, s), FA_ERR_INVALID_ARG);

  if (n_failed) {
    fprintf(stderr, "%d of %d checks failed\n", n_failed, n_checks);
    return 1;
  }
  printf("ok %d\n", n_checks);
  return 0;
}
