// fa_params.h - parameter blocks and launch geometry of the attention kernels, shared
// by the host-side validation (fa_validate.cpp) and the HIP launchers.  Plain C++ with
// no HIP types, so that the validation also builds on its own for host-only tests.
// Internal to the library (not part of the C ABI).
#pragma once

#include <stdint.h>

namespace fa {

// Forward problem description, filled on the host.  Sizes are in elements.
struct FwdParams {
  const uint16_t* q;      // bf16 [B, Sq, H, D]
  const uint16_t* k;      // bf16 [B, Sk, H, D]
  const uint16_t* v;      // bf16 [B, Sk, H, D]
  void* out;              // bf16 [B, Sq, H, D]  or fp32 [S, B, H, Sq, D] (split mode)
  float* lse;             // fp32 [B, H, Sq]     or fp32 [S, B, H, Sq]    (split mode)
  const float* alibi;     // fp32 ALiBi slopes [H] or [B, H], or nullptr
  int alibi_bstride;      // 0: one slope per head for every batch; nheads: [B, H]
  int f16;                // 1: q/k/v/out are fp16, 0: bf16
  int batch, seqlen_q, seqlen_k, nheads;  // varlen: seqlen_q/k are the maximum lengths
  int nheads_k;           // K/V heads; query head h reads K/V head h / (nheads / nheads_k)
  const int* cu_q;        // varlen: [batch + 1] first q/out row of each sequence, or nullptr
  const int* cu_k;        // varlen: [batch + 1] first k/v row of each sequence, or nullptr
  long lse_head_stride;   // varlen: total_q, lse being [nheads, total_q]
  float scale_log2;       // |softmax_scale| * log2(e), or 1 when softmax_scale == 0
  uint32_t q_and;         // 0 when softmax_scale == 0 (Q is zeroed on load), else all ones
  uint32_t q_sign;        // 0x80008000 when softmax_scale < 0 (Q is negated on load), else 0
  int window_left;        // -1 = unbounded
  int window_right;       // -1 = unbounded; already 0 when causal
  int num_q_tiles;        // ceil(Sq / 128)
  int num_splits;         // 1 for the plain forward
  int split_len;          // keys per split (ceil(Sk / num_splits))
  int reverse_q;          // 1: visit the heaviest query tiles first (causal)
  // KV-cache decode (fa_fwd_kvcache); cache_seqlens is nullptr otherwise
  const int* cache_seqlens;  // [batch] rows already in the cache
  const int* block_table;    // [batch, max_blocks] physical block of each logical block, or
                             // nullptr: contiguous cache, block b holds sequence b
  int page_size;             // rows per block (the per-sequence capacity when contiguous)
  int page_shift;            // log2(page_size) when paged
  int max_blocks;            // row length of block_table
  int seqlen_new;            // rows appended to every sequence before the attention
};

// Combine description.
struct CombineParams {
  const float* out_partial;  // [S, B, H, Sq, D]
  const float* lse_partial;  // [S, B, H, Sq]
  uint16_t* out;             // bf16 or fp16 [B, Sq, H, D]
  float* lse;                // [B, H, Sq]
  int batch, seqlen_q, nheads, num_splits;
  int f16;                   // 1: out is fp16, 0: bf16
};

// Backward problem description, filled on the host.  Sizes are in elements.
struct BwdParams {
  const uint16_t* q;      // bf16/fp16 [B, Sq, H, D]
  const uint16_t* k;      // bf16/fp16 [B, Sk, H_k, D]
  const uint16_t* v;      // bf16/fp16 [B, Sk, H_k, D]
  const uint16_t* out;    // bf16/fp16 [B, Sq, H, D]  forward output
  const uint16_t* dout;   // bf16/fp16 [B, Sq, H, D]  upstream gradient
  const float* lse;       // fp32 [B, H, Sq]     forward logsumexp (natural log)
  float* delta;           // fp32 [B, H, Sq]     D, written by dq_kernel, read by dkdv_kernel
  uint16_t* dq;           // bf16/fp16 [B, Sq, H, D]
  uint16_t* dk;           // bf16/fp16 [B, Sk, H_k, D]
  uint16_t* dv;           // bf16/fp16 [B, Sk, H_k, D]
  // Packed batch (cu_q != nullptr): sequence b owns q/dout/dq rows [cu_q[b], cu_q[b+1])
  // and k/v/dk/dv rows [cu_k[b], cu_k[b+1]) of [total, heads, D] tensors; lse and delta
  // are [H, total_q] (lse_head_stride = total_q); seqlen_q/seqlen_k are the maxima.
  const int* cu_q;
  const int* cu_k;
  long lse_head_stride;
  int nheads_k;           // K/V heads; query head h uses K/V head h / (nheads / nheads_k)
  const float* alibi;     // fp32 [H] or [B, H], or nullptr
  int alibi_bstride;      // 0: one slope per head for every batch; nheads: [B, H]
  int f16;                // 1: every 16-bit tensor is fp16, 0: bf16
  int batch, seqlen_q, seqlen_k, nheads;
  float scale;            // softmax_scale as given
  float scale_log2;       // |scale| * log2(e), or 1 when scale == 0
  uint32_t q_and;         // 0 when scale == 0 (the scores are then the bias alone)
  uint32_t q_sign;        // 0x80008000 when scale < 0, else 0
  int window_left, window_right;  // -1 = unbounded; window_right already 0 when causal
  int num_q_tiles;        // ceil(Sq / 128): dq workgroups per (batch, head)
  int num_k_tiles;        // ceil(Sk / 128): dkdv workgroups per (batch, head)
};

// ---- launch geometry ----------------------------------------------------------------

// Matrix-core forward: query rows per workgroup of the default four-wave launch
// (the eight-wave launch has 256-row tiles).
constexpr int FWD_BLOCK_ROWS = 128;
// Backward: rows (queries or keys) a dq / dkdv workgroup owns, 32 per wave.
constexpr int BWD_ROWS = 128;
// Threads per workgroup of every kernel except the eight-wave forward (512).
constexpr int BLOCK_THREADS = 256;

// Eight waves per workgroup (the ping-pong schedule) for the headdim-128 forward with
// neither causal mask nor window from 2048 query rows, and with a plain causal mask
// from 8192; four otherwise.  Measured against four waves (MI355X, 16 heads x 128,
// batch 16384 / seqlen): unmasked +2.5% at 2k, +6-7% at 4k-16k; causal -4% at 2k,
// even at 4k, +5% at 16k.  With ALiBi under a causal mask four waves at every length:
// that kernel runs the key tiles right to left (launch_fwd_hd), +10% at 16k against
// the eight-wave kernel's left-to-right order.
#ifndef FA_EIGHT_WAVE_ROWS
#define FA_EIGHT_WAVE_ROWS 2048
#endif
#ifndef FA_EIGHT_WAVE_CAUSAL_ROWS
#define FA_EIGHT_WAVE_CAUSAL_ROWS 8192
#endif
#ifndef FA_ALIBI_CAUSAL_4W
#define FA_ALIBI_CAUSAL_4W 1
#endif
inline int fwd_waves(int headdim, bool split, int window_left, int window_right, int seqlen_q, bool alibi) {
  if (headdim != 128 || split || window_left >= 0) return 4;
  if (FA_ALIBI_CAUSAL_4W && alibi && window_right == 0) return 4;
  if (window_right < 0) return seqlen_q >= FA_EIGHT_WAVE_ROWS ? 8 : 4;
  return (window_right == 0 && seqlen_q >= FA_EIGHT_WAVE_CAUSAL_ROWS) ? 8 : 4;
}

// The matrix-core decode form serves a KV-cache step whose K/V heads each have more
// than four queries (headdim 64 or 128); the vector-ALU kernel serves the rest.
inline bool decode_uses_mfma(int headdim, int nq_total) { return headdim != 256 && nq_total > 4; }

// Queries one vector-ALU decode workgroup serves when a K/V head has nq_total of them.
inline int decode_queries_per_block(int nq_total) {
  return nq_total <= 1 ? 1 : nq_total <= 2 ? 2 : nq_total <= 4 ? 4 : 8;
}

// Key rows per lane per step of the vector-ALU decode kernel.
#ifndef FA_DEC_UNROLL
#define FA_DEC_UNROLL 8
#endif
constexpr int DEC_UNROLL = FA_DEC_UNROLL;
// Key rows one decode step covers per wave (blocks of a paged cache must hold a whole
// number of them): DEC_UNROLL * 64 / (headdim / 8).
inline int decode_step_keys(int headdim) { return DEC_UNROLL * 64 / (headdim / 8); }

// Size of the device buffer that holds the split partials of fa_fwd_kvcache_noalloc
// (one per GPU, for the life of the process).
#define FA_NOALLOC_SCRATCH_BYTES (16LL << 20)

// A grid's work-item count (workgroups x threads) must fit in 32 bits on this runtime.
inline long long max_grid_blocks(int threads) { return 0xffffffffLL / threads; }

}  // namespace fa
