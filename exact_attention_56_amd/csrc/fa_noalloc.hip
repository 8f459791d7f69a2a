// fa_noalloc.hip - fa_fwd_kvcache_noalloc: the KV-cache decode step of fa_fwd_kvcache
// with its split partials in a library-owned device buffer, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The kernels are fa_fwd_kvcache's, unchanged.
//
// The buffer is the file-scope device array `scratch` below (FA_NOALLOC_SCRATCH_BYTES).
// Every GPU the library runs on holds its own copy until the process ends.  In host
// code the array's name is only a host-side stand-in, so the device address of each
// GPU's copy is looked up once, with hipGetSymbolAddress and that device current, and
// kept per device; kernels receive that address, never the name.  All calls on one GPU
// share the buffer: calls that overlap in time on one GPU (two streams, or two host
// threads) race on it.  Nothing in it needs to start at zero: the partial pass writes
// every row of every split (an empty split writes 0 and -inf) before the combine reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "fa_params.h"
#include "fa_validate.h"

namespace fa {
hipError_t launch_combine(const CombineParams& p, int headdim, hipStream_t stream);
hipError_t launch_kvcache(const FwdParams& p, int headdim, const uint16_t* k_new, const uint16_t* v_new,
                          uint16_t* k_cache, uint16_t* v_cache, const float* cos, const float* sin, int rd,
                          uint16_t* qrot, hipStream_t stream);
}  // namespace fa

static __device__ __align__(256) uint8_t scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on the device that runs `stream`, or nullptr.
void* scratch_address(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int fa_fwd_kvcache_noalloc(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens,
                                      const int* block_table, int page_size, int max_blocks_per_seq,
                                      const void* k_new, const void* v_new, int seqlen_new,
                                      const float* rotary_cos, const float* rotary_sin, int rotary_dim, void* out,
                                      float* lse, int batch, int seqlen_q, int nheads, int nheads_k, int headdim,
                                      float softmax_scale, int causal, int window_left, int window_right,
                                      const float* alibi_slopes, int alibi_per_batch, int dtype, int num_splits,
                                      hipStream_t stream) {
  // the most splits whose partials fit (checked before any HIP call); with
  // num_splits = 0 the automatic count is capped there
  const int max_splits = fa::scratch_max_splits(batch, nheads, seqlen_q, headdim, FA_NOALLOC_SCRATCH_BYTES);
  if (max_splits < 1) return FA_ERR_INVALID_ARG;
  if (num_splits > max_splits) return FA_ERR_INVALID_ARG;
  // Plan against placeholder partial pointers (aligned, never dereferenced) so that
  // every argument is validated before the device buffer is looked up.
  float* const placeholder = (float*)(uintptr_t)256;
  fa::FwdParams p;
  fa::CombineParams c;
  int st = fa::plan_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, block_table, page_size, max_blocks_per_seq, k_new,
                                v_new, seqlen_new, rotary_cos, rotary_sin, rotary_dim, out, lse, placeholder,
                                placeholder, max_splits, batch, seqlen_q, nheads, nheads_k, headdim, softmax_scale,
                                causal, window_left, window_right, alibi_slopes, alibi_per_batch, dtype, num_splits,
                                &p, &c);
  if (st != FA_OK) return st;
  uint8_t* base = (uint8_t*)scratch_address(stream);
  if (base == nullptr) return FA_ERR_LAUNCH;
  // out partials [S, B, H, Sq, D] first, their lse [S, B, H, Sq] after them
  const long long rows = (long long)p.num_splits * batch * nheads * seqlen_q;
  float* out_partial = (float*)base;
  float* lse_partial = (float*)(base + rows * headdim * 4);
  p.out = out_partial;
  p.lse = lse_partial;
  c.out_partial = out_partial;
  c.lse_partial = lse_partial;
  (void)hipGetLastError();
  if (fa::launch_kvcache(p, headdim, (const uint16_t*)k_new, (const uint16_t*)v_new, (uint16_t*)k_cache,
                         (uint16_t*)v_cache, rotary_cos, rotary_sin, rotary_dim, (uint16_t*)out, stream) != hipSuccess)
    return FA_ERR_LAUNCH;
  return fa::launch_combine(c, headdim, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
