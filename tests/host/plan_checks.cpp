// plan_checks.cpp - host-only checks of the C ABI's validation and launch planning
// (exact_attention_56_amd/csrc/fa_validate.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer (no GPU, no HIP calls: the planners touch no device memory).
//
// It checks the derived launch parameters of valid calls, both sides of every grid
// limit (the last grid that fits in 2^32 - 1 work-items is accepted, the next one is
// rejected), and then drives every planner with edge values (0, -1, INT_MAX, INT_MIN,
// powers of two and their neighbours) in every integer argument, so that any signed
// overflow, bad shift or out-of-bounds access in the validation aborts the run.
// Prints "ok <n>" and exits 0 when every check holds.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "fa_validate.h"

static int n_checks = 0, n_failed = 0;

static void expect(long long got, long long want, const char* what, int line) {
  ++n_checks;
  if (got != want) {
    ++n_failed;
    fprintf(stderr, "line %d: %s = %lld, expected %lld\n", line, what, got, want);
  }
}
#define EXPECT(x, want) expect((long long)(x), (long long)(want), #x, __LINE__)

static void* const P = (void*)(uintptr_t)0x100000;
static float* const F = (float*)(uintptr_t)0x200000;
static const int* const I = (const int*)(uintptr_t)0x300000;

static int fwd(int b, int sq, int sk, int h, int d, float scale, int causal, int wl, int wr, fa::FwdParams* p) {
  return fa::plan_fwd(P, P, P, P, F, b, sq, sk, h, d, scale, causal, wl, wr, nullptr, 0, FA_BF16, p);
}

static void derived_fields() {
  fa::FwdParams p;
  // window normalisation: causal wins, sides at least as wide as the range are unbounded
  EXPECT(fwd(2, 300, 500, 4, 128, 0.125f, 1, 600, 7, &p), FA_OK);
  EXPECT(p.window_left, -1);
  EXPECT(p.window_right, 0);
  EXPECT(p.reverse_q, 1);
  EXPECT(p.num_q_tiles, 3);
  EXPECT(fwd(2, 300, 500, 4, 128, 0.125f, 0, 10, 300, &p), FA_OK);
  EXPECT(p.window_left, 10);
  EXPECT(p.window_right, -1);
  EXPECT(p.reverse_q, 0);
  // the scale's sign and zero are folded into Q's load masks
  EXPECT(fwd(1, 4, 4, 1, 64, -0.5f, 0, -1, -1, &p), FA_OK);
  EXPECT(p.q_sign, 0x80008000u);
  EXPECT(p.q_and, 0xffffffffu);
  EXPECT(fabsf(p.scale_log2 - 0.5f * 1.4426950408889634f) < 1e-7f, 1);
  EXPECT(fwd(1, 4, 4, 1, 64, 0.f, 0, -1, -1, &p), FA_OK);
  EXPECT(p.q_and, 0u);
  EXPECT(p.scale_log2 == 1.f, 1);
  // split partials: vector path up to 8 query rows, matrix cores beyond
  int vec = -1;
  EXPECT(fa::plan_fwd_splitkv(P, P, P, F, F, 8, 1, 32768, 16, 128, 0.088f, 1, -1, -1, nullptr, 0, FA_BF16, 16, &p,
                              &vec), FA_OK);
  EXPECT(vec, 1);
  EXPECT(p.split_len, 2048);
  EXPECT(fa::plan_fwd_splitkv(P, P, P, F, F, 1, 9, 1000, 2, 64, 0.1f, 0, -1, -1, nullptr, 0, FA_BF16, 3, &p, &vec),
         FA_OK);
  EXPECT(vec, 0);
  EXPECT(p.split_len, 334);
  // KV-cache: automatic split count (about 2048 one-query workgroups, at least 256 keys)
  fa::CombineParams c;
  EXPECT(fa::plan_fwd_kvcache(P, P, P, I, I, 256, 128, nullptr, nullptr, 0, nullptr, nullptr, 0, P, F, F, F, 64, 8,
                              1, 16, 16, 128, 0.088f, 1, -1, -1, nullptr, 0, FA_BF16, 0, &p, &c), FA_OK);
  EXPECT(p.num_splits, 16);
  EXPECT(c.num_splits, 16);
  EXPECT(p.page_shift, 8);
  EXPECT(p.split_len, 2048);
  // backward tiles
  fa::BwdParams bp;
  EXPECT(fa::plan_bwd(P, P, P, P, F, P, P, P, P, F, 3, 200, 129, 4, 64, 0.125f, 1, -1, -1, nullptr, 0, FA_FP16, &bp),
         FA_OK);
  EXPECT(bp.num_q_tiles, 2);
  EXPECT(bp.num_k_tiles, 2);
  EXPECT(bp.f16, 1);
  EXPECT(bp.window_right, 0);
}

static void grid_limits() {
  fa::FwdParams p;
  fa::CombineParams c;
  fa::BwdParams bp;
  int vec;
  // four-wave forward: 2^24 - 1 workgroups of 256 threads fit, 2^24 do not
  EXPECT(fwd(16777215, 128, 128, 1, 64, 0.1f, 0, -1, -1, &p), FA_OK);
  EXPECT(fwd(16777216, 128, 128, 1, 64, 0.1f, 0, -1, -1, &p), FA_ERR_INVALID_ARG);
  // eight-wave forward (headdim 128, unmasked, >= 4096 rows): 256-row tiles of 512 threads,
  // 2^23 - 1 workgroups fit.  At 4224 rows (17 tiles of 256, 33 of 128) the eight-wave
  // limit binds first: 493447 * 17 = 8388599 fits, 493448 * 17 = 8388616 does not
  EXPECT(fwd(493447, 4224, 4224, 1, 128, 0.1f, 0, -1, -1, &p), FA_OK);
  EXPECT(fwd(493448, 4224, 4224, 1, 128, 0.1f, 0, -1, -1, &p), FA_ERR_INVALID_ARG);
  // the same shape causal runs four-wave workgroups: 493448 * 33 = 16283784 fits
  EXPECT(fwd(493448, 4224, 4224, 1, 128, 0.1f, 1, -1, -1, &p), FA_OK);
  // split partials on the vector path: 2^24 - 1 workgroups fit
  EXPECT(fa::plan_fwd_splitkv(P, P, P, F, F, 16777215, 1, 64, 1, 64, 0.1f, 1, -1, -1, nullptr, 0, FA_BF16, 1, &p,
                              &vec), FA_OK);
  EXPECT(fa::plan_fwd_splitkv(P, P, P, F, F, 16777216, 1, 64, 1, 64, 0.1f, 1, -1, -1, nullptr, 0, FA_BF16, 1, &p,
                              &vec), FA_ERR_INVALID_ARG);
  // combine: one workgroup per row
  EXPECT(fa::plan_combine(F, F, P, F, 1, 16777215, 1, 64, 2, FA_BF16, &c), FA_OK);
  EXPECT(fa::plan_combine(F, F, P, F, 1, 16777216, 1, 64, 2, FA_BF16, &c), FA_ERR_INVALID_ARG);
  // backward: dQ runs one workgroup per 128 query rows, dK/dV one per 128 keys of every
  // (batch, head); each grid holds at most 2^24 - 1 workgroups of 256 threads
  EXPECT(fa::plan_bwd(P, P, P, P, F, P, P, P, P, F, 8388607, 256, 128, 1, 128, 0.1f, 0, -1, -1, nullptr, 0,
                      FA_BF16, &bp), FA_OK);
  EXPECT(fa::plan_bwd(P, P, P, P, F, P, P, P, P, F, 8388608, 256, 128, 1, 128, 0.1f, 0, -1, -1, nullptr, 0,
                      FA_BF16, &bp), FA_ERR_INVALID_ARG);
  EXPECT(fa::plan_bwd(P, P, P, P, F, P, P, P, P, F, 8388608, 128, 256, 1, 64, 0.1f, 0, -1, -1, nullptr, 0,
                      FA_BF16, &bp), FA_ERR_INVALID_ARG);
  EXPECT(fa::plan_bwd(P, P, P, P, F, P, P, P, P, F, 16777215, 128, 128, 1, 256, 0.1f, 0, -1, -1, nullptr, 0,
                      FA_BF16, &bp), FA_OK);
  // KV-cache combine grid: batch * heads * seqlen_q rows
  EXPECT(fa::plan_fwd_kvcache(P, P, P, I, nullptr, 256, 1, nullptr, nullptr, 0, nullptr, nullptr, 0, P, F, F, F, 1,
                              16777215, 1, 1, 1, 64, 0.1f, 1, -1, -1, nullptr, 0, FA_BF16, 1, &p, &c), FA_OK);
  EXPECT(fa::plan_fwd_kvcache(P, P, P, I, nullptr, 256, 1, nullptr, nullptr, 0, nullptr, nullptr, 0, P, F, F, F, 1,
                              16777216, 1, 1, 1, 64, 0.1f, 1, -1, -1, nullptr, 0, FA_BF16, 1, &p, &c),
         FA_ERR_INVALID_ARG);
  // KV-cache preparation grid: four rotated rows per workgroup
  EXPECT(fa::plan_fwd_kvcache(P, P, P, I, nullptr, 256, 1, nullptr, nullptr, 0, F, F, 64, P, F, F, F, 1, 8388607, 8,
                              1, 1, 64, 0.1f, 1, -1, -1, nullptr, 0, FA_BF16, 1, &p, &c), FA_ERR_INVALID_ARG);
}

static void scratch_splits() {
  // 8 x 16 rows of headdim 128: 516 bytes per partial row, 66048 per split
  EXPECT(fa::scratch_max_splits(8, 16, 1, 128, 16LL << 20), 254);
  EXPECT(fa::scratch_max_splits(8, 16, 1, 128, 66048), 1);
  EXPECT(fa::scratch_max_splits(8, 16, 1, 128, 66047), 0);
  EXPECT(fa::scratch_max_splits(0, 16, 1, 128, 1 << 20), 0);
  EXPECT(fa::scratch_max_splits(INT_MAX, INT_MAX, 8, 256, 16LL << 20), 0);
  EXPECT(fa::scratch_max_splits(1, 1, 1, 64, LLONG_MAX), INT_MAX);
}

static const int kEdge[] = {INT_MIN, -65537, -3, -2, -1, 0, 1, 2, 3, 7, 8, 9, 31, 32, 63, 64, 65, 100, 127, 128, 129,
                            255, 256, 257, 4095, 4096, 65535, 65536, 1 << 20, (1 << 24) - 1, 1 << 24,
                            (1 << 30) - 1, 1 << 30, (1 << 30) + 1, INT_MAX - 1, INT_MAX};
static const int kNumEdge = sizeof(kEdge) / sizeof(kEdge[0]);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static int edge() {  // splitmix64 over the edge table
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return kEdge[z % kNumEdge];
}

static void edge_values() {
  const float scales[] = {0.125f, 0.f, -1.f, (float)INFINITY, (float)NAN, 1e30f};
  fa::FwdParams p;
  fa::CombineParams c;
  fa::BwdParams bp;
  int vec;
  long long accepted = 0, calls = 0;
  for (int it = 0; it < 40000; ++it) {
    const float sc = scales[it % 6];
    int st;
    st = fa::plan_fwd(P, P, P, P, F, edge(), edge(), edge(), edge(), edge(), sc, it & 1, edge(), edge(), nullptr, 0,
                      FA_BF16, &p);
    accepted += st == FA_OK;
    st = fa::plan_fwd_splitkv(P, P, P, F, F, edge(), edge(), edge(), edge(), edge(), sc, it & 1, edge(), edge(), F,
                              it & 1, FA_FP16, edge(), &p, &vec);
    accepted += st == FA_OK;
    st = fa::plan_fwd_varlen(P, P, P, P, F, I, I, edge(), edge(), edge(), edge(), edge(), edge(), edge(), sc, it & 1,
                             edge(), edge(), nullptr, 0, FA_BF16, &p);
    accepted += st == FA_OK;
    st = fa::plan_combine(F, F, P, F, edge(), edge(), edge(), edge(), edge(), it & 1, &c);
    accepted += st == FA_OK;
    st = fa::plan_fwd_kvcache(P, P, P, I, (it & 2) ? I : nullptr, edge(), edge(), P, P, edge(), (it & 4) ? F : nullptr,
                              (it & 4) ? F : nullptr, edge(), P, F, F, F, edge(), edge(), edge(), edge(), edge(),
                              edge(), sc, it & 1, edge(), edge(), nullptr, 0, FA_BF16, edge(), &p, &c);
    accepted += st == FA_OK;
    st = fa::plan_bwd(P, P, P, P, F, P, P, P, P, F, edge(), edge(), edge(), edge(), edge(), sc, it & 1, edge(), edge(),
                      nullptr, 0, FA_BF16, &bp);
    accepted += st == FA_OK;
    st = fa::plan_bwd_varlen(P, P, P, P, F, P, P, P, P, F, I, I, edge(), edge(), edge(), edge(), edge(), edge(),
                             edge(), edge(), sc, it & 1, edge(), edge(), nullptr, 0, FA_BF16, &bp);
    accepted += st == FA_OK;
    calls += 7;
  }
  // the sweep reached both outcomes
  EXPECT(accepted > 0, 1);
  EXPECT(accepted < calls, 1);
}

int main() {
  derived_fields();
  grid_limits();
  scratch_splits();
  edge_values();
  if (n_failed) {
    fprintf(stderr, "%d of %d checks failed\n", n_failed, n_checks);
    return 1;
  }
  printf("ok %d\n", n_checks);
  return 0;
}
