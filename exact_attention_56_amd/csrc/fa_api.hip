// fa_api.hip - the extern "C" entry points declared in include/fa.h.
//
// Each entry point first runs its plan (fa_validate.cpp): every argument and every
// grid of the call is checked before any HIP call, so an invalid call launches
// nothing and touches no output.  Then it launches on the caller's stream, checking
// the runtime's status after each launch before the next.  No allocation, no
// synchronisation, no global state.
#include "fa.h"
#include "fa_bwd_kernel.h"
#include "fa_validate.h"

namespace fa {
hipError_t launch_fwd(const FwdParams& p, int headdim, bool split, hipStream_t stream);
hipError_t launch_decode(const FwdParams& p, int headdim, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, int headdim, hipStream_t stream);
hipError_t launch_kvcache(const FwdParams& p, int headdim, const uint16_t* k_new, const uint16_t* v_new,
                          uint16_t* k_cache, uint16_t* v_cache, const float* cos, const float* sin, int rd,
                          uint16_t* qrot, hipStream_t stream);
}  // namespace fa

namespace {
int launched(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }
}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int seqlen_q,
           int seqlen_k, int nheads, int headdim, float softmax_scale, int causal, int window_left,
           int window_right, const float* alibi_slopes, int alibi_per_batch, int dtype, hipStream_t stream) {
  fa::FwdParams p;
  const int st = fa::plan_fwd(q, k, v, out, lse, batch, seqlen_q, seqlen_k, nheads, headdim, softmax_scale, causal,
                              window_left, window_right, alibi_slopes, alibi_per_batch, dtype, &p);
  if (st != FA_OK) return st;
  (void)hipGetLastError();  // clear a stale error so the check below sees this launch only
  return launched(fa::launch_fwd(p, headdim, false, stream));
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, float* out_partial, float* lse_partial,
                   int batch, int seqlen_q, int seqlen_k, int nheads, int headdim, float softmax_scale,
                   int causal, int window_left, int window_right, const float* alibi_slopes,
                   int alibi_per_batch, int dtype, int num_splits, hipStream_t stream) {
  fa::FwdParams p;
  int vector_path = 0;
  const int st = fa::plan_fwd_splitkv(q, k, v, out_partial, lse_partial, batch, seqlen_q, seqlen_k, nheads, headdim,
                                      softmax_scale, causal, window_left, window_right, alibi_slopes,
                                      alibi_per_batch, dtype, num_splits, &p, &vector_path);
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  return launched(vector_path ? fa::launch_decode(p, headdim, stream) : fa::launch_fwd(p, headdim, true, stream));
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int batch, int max_seqlen_q, int max_seqlen_k, int total_q, int nheads,
                  int nheads_k, int headdim, float softmax_scale, int causal, int window_left, int window_right,
                  const float* alibi_slopes, int alibi_per_batch, int dtype, hipStream_t stream) {
  fa::FwdParams p;
  const int st = fa::plan_fwd_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q,
                                     max_seqlen_k, total_q, nheads, nheads_k, headdim, softmax_scale, causal,
                                     window_left, window_right, alibi_slopes, alibi_per_batch, dtype, &p);
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  return launched(fa::launch_fwd(p, headdim, false, stream));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* delta, int batch, int seqlen_q, int seqlen_k, int nheads,
           int headdim, float softmax_scale, int causal, int window_left, int window_right,
           const float* alibi_slopes, int alibi_per_batch, int dtype, hipStream_t stream) {
  fa::BwdParams p;
  const int st = fa::plan_bwd(q, k, v, out, lse, dout, dq, dk, dv, delta, batch, seqlen_q, seqlen_k, nheads, headdim,
                              softmax_scale, causal, window_left, window_right, alibi_slopes, alibi_per_batch, dtype,
                              &p);
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  return launched(fa::launch_bwd(p, headdim, stream));
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int batch, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int nheads, int nheads_k,
                  int headdim, float softmax_scale, int causal, int window_left, int window_right,
                  const float* alibi_slopes, int alibi_per_batch, int dtype, hipStream_t stream) {
  fa::BwdParams p;
  const int st = fa::plan_bwd_varlen(q, k, v, out, lse, dout, dq, dk, dv, delta, cu_seqlens_q, cu_seqlens_k, batch,
                                     max_seqlen_q, max_seqlen_k, total_q, total_k, nheads, nheads_k, headdim,
                                     softmax_scale, causal, window_left, window_right, alibi_slopes, alibi_per_batch,
                                     dtype, &p);
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  return launched(fa::launch_bwd(p, headdim, stream));
}

int fa_fwd_kvcache(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens, const int* block_table,
                   int page_size, int max_blocks_per_seq, const void* k_new, const void* v_new, int seqlen_new,
                   const float* rotary_cos, const float* rotary_sin, int rotary_dim, void* out, float* lse,
                   float* out_partial, float* lse_partial, int max_splits, int batch, int seqlen_q, int nheads,
                   int nheads_k, int headdim, float softmax_scale, int causal, int window_left, int window_right,
                   const float* alibi_slopes, int alibi_per_batch, int dtype, int num_splits,
                   hipStream_t stream) {
  fa::FwdParams p;
  fa::CombineParams c;
  const int st = fa::plan_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, block_table, page_size, max_blocks_per_seq,
                                      k_new, v_new, seqlen_new, rotary_cos, rotary_sin, rotary_dim, out, lse,
                                      out_partial, lse_partial, max_splits, batch, seqlen_q, nheads, nheads_k,
                                      headdim, softmax_scale, causal, window_left, window_right, alibi_slopes,
                                      alibi_per_batch, dtype, num_splits, &p, &c);
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  if (fa::launch_kvcache(p, headdim, (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)k_cache,
                         (uint16_t*)v_cache, rotary_cos, rotary_sin, rotary_dim, (uint16_t*)out, stream) != hipSuccess)
    return FA_ERR_LAUNCH;
  return launched(fa::launch_combine(c, headdim, stream));
}

int fa_combine(const float* out_partial, const float* lse_partial, void* out, float* lse, int batch,
               int seqlen_q, int nheads, int headdim, int num_splits, int dtype, hipStream_t stream) {
  fa::CombineParams p;
  const int st = fa::plan_combine(out_partial, lse_partial, out, lse, batch, seqlen_q, nheads, headdim, num_splits,
                                  dtype, &p);
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  return launched(fa::launch_combine(p, headdim, stream));
}

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: headdim must be 64, 128 or 256";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime rejected the kernel launch";
    default: return "unknown status";
  }
}

}  // extern "C"
