// fa_validate.h - host-side validation and launch planning of the C ABI entry points.
//
// Each plan_* function checks every argument of one entry point of include/fa.h,
// including the size of every grid the call will launch, and on success fills the
// kernel parameter blocks; it returns FA_OK or the entry point's error code and
// touches no device memory.  The entry points (fa_api.hip) launch only after their
// plan succeeded, so an invalid call launches nothing.  Plain C++ (no HIP calls):
// it also builds on its own for the host-only sanitizer test.
#pragma once

#include "fa.h"
#include "fa_params.h"

namespace fa {

int plan_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int seqlen_q,
             int seqlen_k, int nheads, int headdim, float softmax_scale, int causal, int window_left,
             int window_right, const float* alibi_slopes, int alibi_per_batch, int dtype, FwdParams* p);

// *vector_path: 1 when the split partials run on the vector-ALU decode kernel
// (seqlen_q <= 8), 0 for the matrix-core kernel in split mode.
int plan_fwd_splitkv(const void* q, const void* k, const void* v, float* out_partial, float* lse_partial,
                     int batch, int seqlen_q, int seqlen_k, int nheads, int headdim, float softmax_scale,
                     int causal, int window_left, int window_right, const float* alibi_slopes, int alibi_per_batch,
                     int dtype, int num_splits, FwdParams* p, int* vector_path);

int plan_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                    int nheads, int nheads_k, int headdim, float softmax_scale, int causal, int window_left,
                    int window_right, const float* alibi_slopes, int alibi_per_batch, int dtype, FwdParams* p);

int plan_combine(const float* out_partial, const float* lse_partial, void* out, float* lse, int batch,
                 int seqlen_q, int nheads, int headdim, int num_splits, int dtype, CombineParams* p);

// Fills the partial pass (p) and the combine (c) of a KV-cache step; num_splits = 0
// picks the split count.
int plan_fwd_kvcache(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens, const int* block_table,
                     int page_size, int max_blocks_per_seq, const void* k_new, const void* v_new, int seqlen_new,
                     const float* rotary_cos, const float* rotary_sin, int rotary_dim, void* out, float* lse,
                     float* out_partial, float* lse_partial, int max_splits, int batch, int seqlen_q, int nheads,
                     int nheads_k, int headdim, float softmax_scale, int causal, int window_left, int window_right,
                     const float* alibi_slopes, int alibi_per_batch, int dtype, int num_splits, FwdParams* p,
                     CombineParams* c);

// Most splits whose partials (fp32 out [S, B, H, Sq, D] followed by lse [S, B, H, Sq])
// fit in `bytes`; 0 when not even one split fits or a size is not positive.
int scratch_max_splits(int batch, int nheads, int seqlen_q, int headdim, long long bytes);

int plan_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* delta, int batch, int seqlen_q, int seqlen_k, int nheads,
             int headdim, float softmax_scale, int causal, int window_left, int window_right,
             const float* alibi_slopes, int alibi_per_batch, int dtype, BwdParams* p);

int plan_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* delta, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k, int total_q,
                    int total_k, int nheads, int nheads_k, int headdim, float softmax_scale, int causal,
                    int window_left, int window_right, const float* alibi_slopes, int alibi_per_batch, int dtype,
                    BwdParams* p);

}  // namespace fa
