// fa_validate.cpp - host-side validation and launch planning of the C ABI entry points
// (declared in fa_validate.h).  Plain C++: no HIP calls, no device memory touched.
#include "fa_validate.h"

#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

namespace fa {
namespace {

constexpr int kMaxSeqlen = 1 << 30;          // keeps every position/window sum inside int32
constexpr int kDecodeMaxRows = 8;            // fa_fwd_splitkv: vector-ALU path up to this seqlen_q
constexpr long long kMaxRowElems = 1 << 22;  // nheads * headdim
constexpr float kLog2eHost = 1.4426950408889634f;

bool headdim_supported(int d) { return d == 64 || d == 128 || d == 256; }

// Elements of a [a, b, c, d] tensor, or -1 when it does not fit in int64.
long long elems4(long long a, long long b, long long c, long long d) {
  long long r = 1;
  const long long f[4] = {a, b, c, d};
  for (long long x : f) {
    if (x <= 0 || r > (long long)INT64_MAX / 2 / x) return -1;
    r *= x;
  }
  return r;
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// A grid of `blocks` workgroups of `threads` threads fits the runtime's 32-bit
// work-item count (and the kernels' int item indices).
bool grid_ok(long long blocks, int threads) { return blocks >= 1 && blocks <= max_grid_blocks(threads); }

// 16-bit tensors start on a 16-byte boundary (the kernels move 16 bytes per lane);
// a NULL optional pointer passes.
bool aligned16(const void* x) { return ((uintptr_t)x & 15) == 0; }

// Validation shared by every entry point that takes q, k, v and the mask arguments.
// Fills p (everything but the outputs) on success.
int prepare(const void* q, const void* k, const void* v, int batch, int seqlen_q, int seqlen_k, int nheads,
            int headdim, float softmax_scale, int causal, int window_left, int window_right,
            const float* alibi_slopes, int alibi_per_batch, int dtype, FwdParams* p) {
  if (!q || !k || !v) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_INVALID_ARG;
  if (alibi_per_batch != 0 && alibi_per_batch != 1) return FA_ERR_INVALID_ARG;
  if (batch < 1 || seqlen_q < 1 || seqlen_k < 1 || nheads < 1 || headdim < 1) return FA_ERR_INVALID_ARG;
  if (seqlen_q > kMaxSeqlen || seqlen_k > kMaxSeqlen) return FA_ERR_INVALID_ARG;
  if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale)) return FA_ERR_INVALID_ARG;
  if (!headdim_supported(headdim)) return FA_ERR_UNSUPPORTED;
  if (elems4(batch, seqlen_q, nheads, headdim) < 0 || elems4(batch, seqlen_k, nheads, headdim) < 0)
    return FA_ERR_INVALID_ARG;
  // The kernels address at most 128 key rows (nheads*headdim 16-bit values apart) from
  // one buffer base with 32-bit offsets.
  if ((long long)nheads * headdim > kMaxRowElems) return FA_ERR_UNSUPPORTED;

  int wl = window_left;
  int wr = causal ? 0 : window_right;
  // A side at least as wide as the whole key range is the same as no bound:
  // c_i - wl < 0 <= j for every row when wl >= Sk, and c_i + wr >= Sk - 1 >= j
  // for every row when wr >= Sq.
  if (wl >= seqlen_k) wl = -1;
  if (wr >= seqlen_q) wr = -1;

  p->q = (const uint16_t*)q;
  p->k = (const uint16_t*)k;
  p->v = (const uint16_t*)v;
  p->out = nullptr;
  p->lse = nullptr;
  p->alibi = alibi_slopes;
  p->alibi_bstride = alibi_per_batch ? nheads : 0;
  p->f16 = dtype == FA_FP16 ? 1 : 0;
  p->batch = batch;
  p->seqlen_q = seqlen_q;
  p->seqlen_k = seqlen_k;
  p->nheads = nheads;
  p->nheads_k = nheads;
  p->cu_q = nullptr;
  p->cu_k = nullptr;
  p->lse_head_stride = 0;
  p->cache_seqlens = nullptr;
  p->block_table = nullptr;
  p->page_size = 0;
  p->page_shift = 0;
  p->max_blocks = 0;
  p->seqlen_new = 0;
  // The kernels fold the scale into Q's sign and a positive multiplier: a negative
  // scale negates Q, a zero scale zeroes Q (every score is then exactly 0).
  if (softmax_scale == 0.f) {
    p->scale_log2 = 1.f;
    p->q_and = 0u;
    p->q_sign = 0u;
  } else {
    p->scale_log2 = fabsf(softmax_scale) * kLog2eHost;
    p->q_and = 0xffffffffu;
    p->q_sign = signbit(softmax_scale) ? 0x80008000u : 0u;
  }
  p->window_left = wl;
  p->window_right = wr;
  p->num_q_tiles = (int)ceil_div(seqlen_q, FWD_BLOCK_ROWS);
  p->num_splits = 1;
  p->split_len = seqlen_k;
  // Causal (or a right window): later query tiles see more keys; start them first.
  p->reverse_q = (wr >= 0) ? 1 : 0;
  return FA_OK;
}

// Grid of the matrix-core forward over p (eight-wave launches use 256-row tiles).
bool fwd_grid_ok(const FwdParams& p, int headdim, bool split) {
  const int nw = fwd_waves(headdim, split, p.window_left, p.window_right, p.seqlen_q, p.alibi != nullptr);
  const long long tiles = ceil_div(p.seqlen_q, 32 * nw);
  return grid_ok((long long)p.batch * p.nheads * tiles * (split ? p.num_splits : 1), 64 * nw);
}

// Copies the forward's validated fields into a backward parameter block.
void bwd_from_fwd(const FwdParams& f, float softmax_scale, const void* out, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta, BwdParams* p) {
  p->q = f.q;
  p->k = f.k;
  p->v = f.v;
  p->out = (const uint16_t*)out;
  p->dout = (const uint16_t*)dout;
  p->lse = lse;
  p->delta = delta;
  p->dq = (uint16_t*)dq;
  p->dk = (uint16_t*)dk;
  p->dv = (uint16_t*)dv;
  p->alibi = f.alibi;
  p->alibi_bstride = f.alibi_bstride;
  p->f16 = f.f16;
  p->batch = f.batch;
  p->seqlen_q = f.seqlen_q;
  p->seqlen_k = f.seqlen_k;
  p->nheads = f.nheads;
  p->nheads_k = f.nheads_k;
  p->cu_q = nullptr;
  p->cu_k = nullptr;
  p->lse_head_stride = 0;
  p->scale = softmax_scale;
  p->scale_log2 = f.scale_log2;
  p->q_and = f.q_and;
  p->q_sign = f.q_sign;
  p->window_left = f.window_left;
  p->window_right = f.window_right;
  p->num_q_tiles = (int)ceil_div(f.seqlen_q, BWD_ROWS);
  p->num_k_tiles = (int)ceil_div(f.seqlen_k, BWD_ROWS);
}

// The two grids of the backward: dK/dV over key tiles of every K/V head, dQ over query
// tiles of every query head.
bool bwd_grids_ok(const BwdParams& p) {
  return grid_ok((long long)p.batch * p.nheads_k * p.num_k_tiles, BLOCK_THREADS) &&
         grid_ok((long long)p.batch * p.nheads * p.num_q_tiles, BLOCK_THREADS);
}

}  // namespace

int plan_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int seqlen_q,
             int seqlen_k, int nheads, int headdim, float softmax_scale, int causal, int window_left,
             int window_right, const float* alibi_slopes, int alibi_per_batch, int dtype, FwdParams* p) {
  if (!out || !lse || !aligned16(out)) return FA_ERR_INVALID_ARG;
  const int st = prepare(q, k, v, batch, seqlen_q, seqlen_k, nheads, headdim, softmax_scale, causal, window_left,
                         window_right, alibi_slopes, alibi_per_batch, dtype, p);
  if (st != FA_OK) return st;
  p->out = out;
  p->lse = lse;
  return fwd_grid_ok(*p, headdim, false) ? FA_OK : FA_ERR_INVALID_ARG;
}

int plan_fwd_splitkv(const void* q, const void* k, const void* v, float* out_partial, float* lse_partial,
                     int batch, int seqlen_q, int seqlen_k, int nheads, int headdim, float softmax_scale,
                     int causal, int window_left, int window_right, const float* alibi_slopes, int alibi_per_batch,
                     int dtype, int num_splits, FwdParams* p, int* vector_path) {
  if (!out_partial || !lse_partial || !aligned16(out_partial)) return FA_ERR_INVALID_ARG;
  const int st = prepare(q, k, v, batch, seqlen_q, seqlen_k, nheads, headdim, softmax_scale, causal, window_left,
                         window_right, alibi_slopes, alibi_per_batch, dtype, p);
  if (st != FA_OK) return st;
  if (num_splits < 1 || num_splits > seqlen_k) return FA_ERR_INVALID_ARG;
  if (elems4(num_splits, batch, (long long)nheads * seqlen_q, headdim) < 0) return FA_ERR_INVALID_ARG;
  p->out = out_partial;
  p->lse = lse_partial;
  p->num_splits = num_splits;
  p->split_len = (int)ceil_div(seqlen_k, num_splits);
  *vector_path = seqlen_q <= kDecodeMaxRows ? 1 : 0;
  if (*vector_path) {
    // one workgroup per (batch, head, split, chunk of up to eight queries)
    const long long chunks = ceil_div(seqlen_q, decode_queries_per_block(seqlen_q));
    if (!grid_ok((long long)batch * nheads * num_splits * chunks, BLOCK_THREADS)) return FA_ERR_INVALID_ARG;
  } else if (!fwd_grid_ok(*p, headdim, true)) {
    return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

int plan_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                    int nheads, int nheads_k, int headdim, float softmax_scale, int causal, int window_left,
                    int window_right, const float* alibi_slopes, int alibi_per_batch, int dtype, FwdParams* p) {
  if (!out || !lse || !cu_seqlens_q || !cu_seqlens_k || !aligned16(out)) return FA_ERR_INVALID_ARG;
  if (nheads_k < 1 || nheads < 1 || nheads % nheads_k != 0 || total_q < 1) return FA_ERR_INVALID_ARG;
  // The per-sequence lengths live on the device; the maxima size the grid and the
  // window normalisation.  One padded "batch" of max_seqlen rows is validated in
  // their place (every sequence is at most that long).
  const int st = prepare(q, k, v, 1, max_seqlen_q, max_seqlen_k, nheads, headdim, softmax_scale, causal,
                         window_left, window_right, alibi_slopes, alibi_per_batch, dtype, p);
  if (st != FA_OK) return st;
  if (batch < 1 || elems4(total_q, nheads, headdim, 1) < 0) return FA_ERR_INVALID_ARG;
  p->batch = batch;
  p->nheads_k = nheads_k;
  p->cu_q = cu_seqlens_q;
  p->cu_k = cu_seqlens_k;
  p->lse_head_stride = total_q;
  p->out = out;
  p->lse = lse;
  return fwd_grid_ok(*p, headdim, false) ? FA_OK : FA_ERR_INVALID_ARG;
}

int plan_combine(const float* out_partial, const float* lse_partial, void* out, float* lse, int batch,
                 int seqlen_q, int nheads, int headdim, int num_splits, int dtype, CombineParams* p) {
  if (!out_partial || !lse_partial || !out || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(out_partial) || !aligned16(out)) return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_INVALID_ARG;
  if (batch < 1 || seqlen_q < 1 || nheads < 1 || headdim < 1 || num_splits < 1) return FA_ERR_INVALID_ARG;
  if (seqlen_q > kMaxSeqlen) return FA_ERR_INVALID_ARG;
  if (!headdim_supported(headdim)) return FA_ERR_UNSUPPORTED;
  if (elems4(num_splits, batch, (long long)nheads * seqlen_q, headdim) < 0) return FA_ERR_INVALID_ARG;
  // one workgroup per row
  if (!grid_ok((long long)batch * nheads * seqlen_q, BLOCK_THREADS)) return FA_ERR_INVALID_ARG;
  p->out_partial = out_partial;
  p->lse_partial = lse_partial;
  p->out = (uint16_t*)out;
  p->lse = lse;
  p->batch = batch;
  p->seqlen_q = seqlen_q;
  p->nheads = nheads;
  p->num_splits = num_splits;
  p->f16 = dtype == FA_FP16 ? 1 : 0;
  return FA_OK;
}

int plan_fwd_kvcache(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens, const int* block_table,
                     int page_size, int max_blocks_per_seq, const void* k_new, const void* v_new, int seqlen_new,
                     const float* rotary_cos, const float* rotary_sin, int rotary_dim, void* out, float* lse,
                     float* out_partial, float* lse_partial, int max_splits, int batch, int seqlen_q, int nheads,
                     int nheads_k, int headdim, float softmax_scale, int causal, int window_left, int window_right,
                     const float* alibi_slopes, int alibi_per_batch, int dtype, int num_splits, FwdParams* p,
                     CombineParams* c) {
  if (!cache_seqlens || !out || !lse || !out_partial || !lse_partial) return FA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(out_partial) || !aligned16(k_new) || !aligned16(v_new)) return FA_ERR_INVALID_ARG;
  if (seqlen_q < 1 || seqlen_q > kDecodeMaxRows || seqlen_new < 0 || page_size < 1 || max_splits < 1)
    return FA_ERR_INVALID_ARG;
  if (nheads < 1 || nheads_k < 1 || nheads % nheads_k != 0) return FA_ERR_INVALID_ARG;
  if (seqlen_new > 0 && (!k_new || !v_new)) return FA_ERR_INVALID_ARG;
  if ((rotary_cos == nullptr) != (rotary_sin == nullptr)) return FA_ERR_INVALID_ARG;
  if (rotary_cos && (rotary_dim < 2 || rotary_dim % 2 != 0 || rotary_dim > headdim)) return FA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > max_splits) return FA_ERR_INVALID_ARG;
  if (!headdim_supported(headdim)) return FA_ERR_UNSUPPORTED;
  int shift = 0;
  long long capacity = page_size;
  if (block_table) {
    // a decode step never crosses a block: blocks are a power of two of at least 64 rows
    if ((page_size & (page_size - 1)) != 0 || page_size < 64 || page_size % decode_step_keys(headdim) != 0 ||
        max_blocks_per_seq < 1)
      return FA_ERR_INVALID_ARG;
    while ((1 << shift) < page_size) ++shift;
    capacity = (long long)page_size * max_blocks_per_seq;
  }
  if (capacity > kMaxSeqlen) return FA_ERR_INVALID_ARG;
  if (seqlen_new > capacity) return FA_ERR_INVALID_ARG;
  const int st = prepare(q, k_cache, v_cache, batch, seqlen_q, (int)capacity, nheads, headdim, softmax_scale,
                         causal, window_left, window_right, alibi_slopes, alibi_per_batch, dtype, p);
  if (st != FA_OK) return st;
  if (elems4(batch, seqlen_new > 0 ? seqlen_new : 1, nheads_k, headdim) < 0) return FA_ERR_INVALID_ARG;
  const int nq = nheads / nheads_k * seqlen_q;  // queries per K/V head
  const bool mfma = decode_uses_mfma(headdim, nq);
  const int per_block = mfma ? FWD_BLOCK_ROWS : decode_queries_per_block(nq);
  const long long chunks = ceil_div(nq, per_block);  // workgroups per (batch, K/V head, split)
  // automatic split count, at least 256 keys per split.  A workgroup serves up to eight
  // queries of one K/V head.  Workgroups of one or two queries are short: about 2048 of
  // them (eight per CU) keep HBM busy.  Workgroups of four or eight queries do four to
  // eight times the work per key: about 512 measured best (paged 32k-key caches, batch 8:
  // +7% at four queries, +35-40% at eight, against 2048).
  int ns = num_splits;
  if (ns == 0) {
    const long long rows = (long long)batch * nheads_k * chunks;
    const long long target = nq >= 3 ? 512 : 2048;
    ns = (int)std::min<long long>(max_splits, std::max<long long>(1, ceil_div(target, rows)));
    ns = (int)std::min<long long>(ns, std::max<long long>(1, capacity / 256));
  }
  if (elems4(ns, batch, (long long)nheads * seqlen_q, headdim) < 0) return FA_ERR_INVALID_ARG;
  // the grids: cache preparation (four rows per workgroup: appended rows, and the
  // queries when rotated), the split partials, the combine (one workgroup per row)
  const long long prep_rows =
      (long long)batch * seqlen_new * nheads_k + (rotary_cos ? (long long)batch * seqlen_q * nheads : 0);
  if (prep_rows > 0 && !grid_ok(ceil_div(prep_rows, 4), BLOCK_THREADS)) return FA_ERR_INVALID_ARG;
  if (!grid_ok((long long)batch * nheads_k * ns * chunks, BLOCK_THREADS)) return FA_ERR_INVALID_ARG;
  if (!grid_ok((long long)batch * nheads * seqlen_q, BLOCK_THREADS)) return FA_ERR_INVALID_ARG;
  p->nheads_k = nheads_k;
  p->cache_seqlens = cache_seqlens;
  p->block_table = block_table;
  p->page_size = page_size;
  p->page_shift = shift;
  p->max_blocks = block_table ? max_blocks_per_seq : 1;
  p->seqlen_new = seqlen_new;
  p->out = out_partial;
  p->lse = lse_partial;
  p->num_splits = ns;
  p->split_len = (int)ceil_div(capacity, ns);
  c->out_partial = out_partial;
  c->lse_partial = lse_partial;
  c->out = (uint16_t*)out;
  c->lse = lse;
  c->batch = batch;
  c->seqlen_q = seqlen_q;
  c->nheads = nheads;
  c->num_splits = ns;
  c->f16 = p->f16;
  return FA_OK;
}

int scratch_max_splits(int batch, int nheads, int seqlen_q, int headdim, long long bytes) {
  if (batch < 1 || nheads < 1 || seqlen_q < 1 || headdim < 1 || bytes < 1) return 0;
  const long long row_bytes = 4LL * headdim + 4;  // one partial row and its lse
  const long long rows = elems4(batch, nheads, seqlen_q, 1);
  if (rows < 0 || rows > bytes / row_bytes) return 0;
  return (int)std::min<long long>(INT_MAX, bytes / (rows * row_bytes));
}

int plan_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* delta, int batch, int seqlen_q, int seqlen_k, int nheads,
             int headdim, float softmax_scale, int causal, int window_left, int window_right,
             const float* alibi_slopes, int alibi_per_batch, int dtype, BwdParams* p) {
  if (!out || !lse || !dout || !dq || !dk || !dv || !delta) return FA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  FwdParams f;  // the forward's validation and window normalisation
  const int st = prepare(q, k, v, batch, seqlen_q, seqlen_k, nheads, headdim, softmax_scale, causal, window_left,
                         window_right, alibi_slopes, alibi_per_batch, dtype, &f);
  if (st != FA_OK) return st;
  bwd_from_fwd(f, softmax_scale, out, lse, dout, dq, dk, dv, delta, p);
  return bwd_grids_ok(*p) ? FA_OK : FA_ERR_INVALID_ARG;
}

int plan_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* delta, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                    int total_k, int nheads, int nheads_k, int headdim, float softmax_scale, int causal,
                    int window_left, int window_right, const float* alibi_slopes, int alibi_per_batch, int dtype,
                    BwdParams* p) {
  if (!out || !lse || !dout || !dq || !dk || !dv || !delta || !cu_seqlens_q || !cu_seqlens_k)
    return FA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  if (nheads_k < 1 || nheads < 1 || nheads % nheads_k != 0 || total_q < 1 || total_k < 1 || batch < 1)
    return FA_ERR_INVALID_ARG;
  // As in fa_fwd_varlen: one padded sequence of the maximal lengths is validated in
  // place of the device-resident per-sequence lengths.
  FwdParams f;
  const int st = prepare(q, k, v, 1, max_seqlen_q, max_seqlen_k, nheads, headdim, softmax_scale, causal,
                         window_left, window_right, alibi_slopes, alibi_per_batch, dtype, &f);
  if (st != FA_OK) return st;
  if (elems4(total_q, nheads, headdim, 1) < 0 || elems4(total_k, nheads_k, headdim, 1) < 0) return FA_ERR_INVALID_ARG;
  f.batch = batch;
  f.nheads_k = nheads_k;
  bwd_from_fwd(f, softmax_scale, out, lse, dout, dq, dk, dv, delta, p);
  p->cu_q = cu_seqlens_q;
  p->cu_k = cu_seqlens_k;
  p->lse_head_stride = total_q;
  return bwd_grids_ok(*p) ? FA_OK : FA_ERR_INVALID_ARG;
}

}  // namespace fa
