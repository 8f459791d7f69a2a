/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention library, libfa_mi355x.so.
 *
 * The library computes exact scaled-dot-product attention,
 *     out = softmax(Q K^T * softmax_scale + mask + ALiBi bias) V,
 * tile by tile with an online softmax, so the seqlen_q x seqlen_k score matrix
 * never reaches device memory, and writes the row-wise logsumexp as well; the
 * split-KV pair and the KV-cache entry serve decoding, and fa_bwd the gradients.
 * Sources (web pages, cited by title and section):
 *   [FA-overview] "FlashAttention：快速且内存高效的准确注意力机制"
 *                 (cloud.tencent.com.cn/developer/article/2433927)
 *     section "使用示例"       : the computation softmax(Q K^T * softmax_scale) V, exact;
 *     section "参数说明"       : argument meanings (softmax_scale default 1/sqrt(headdim),
 *                                window_size (left, right) with -1 = unbounded, fp32
 *                                alibi_slopes adding -slope * |i - j| to score (i, j));
 *     section "算法 / 前向传播": unscaled running output, one final division by the
 *                                row sum, and the row-wise logsumexp L as a second output;
 *     section "2.1：更改causal标志的行为": causal mask aligned to the bottom-right corner
 *                                when seqlen_q != seqlen_k; an all-masked row gives zeros;
 *     section "2.2：针对推理进行优化": for very short queries the KV cache is split over
 *                                workgroups and a separate kernel merges the results;
 *     section "2.3：局部（即滑动窗口）注意力": sliding-window local attention;
 *     section "2.4：ALiBi": ALiBi slopes, one per head or one per (batch, head).
 *   The interface's dtype checks ("代码解读：FlashSelfAttention") accept fp16 and bf16.
 *
 * Conventions shared by every entry point
 *   - q, k, v, out: 16-bit floating point, contiguous [batch, seqlen, nheads, headdim],
 *     headdim innermost.  q and out have seqlen_q rows, k and v have seqlen_k rows,
 *     same nheads.  `dtype` names the element type of every such tensor of a call
 *     (the gradients of fa_bwd and the KV cache included): FA_BF16 or FA_FP16.  The
 *     arithmetic is the same for both: fp32 accumulation, the probabilities rounded
 *     to dtype for the P V product, the output rounded to dtype (nearest even).
 *     Every such tensor (q, k, v, out, the cache and appended rows, dout, dq, dk, dv),
 *     and the fp32 split partials out_partial, starts on a 16-byte boundary: the
 *     kernels move 16 bytes per lane.
 *   - lse: fp32, contiguous [batch, nheads, seqlen_q], natural logarithm of
 *     sum_j exp(softmax_scale * q_i . k_j + bias_ij) over the visible keys.
 *   - Visibility (bottom-right alignment): query i sits at key position
 *     c_i = i + seqlen_k - seqlen_q.  Key j is visible iff
 *         (window_left  < 0 || j >= c_i - window_left) &&
 *         (window_right < 0 || j <= c_i + window_right),
 *     bounds inclusive; causal != 0 sets window_right to 0 (causal wins).
 *   - ALiBi: alibi_slopes is NULL (no bias) or a device fp32 array, [nheads] when
 *     alibi_per_batch is 0 and [batch, nheads] when it is 1 (for fa_fwd_varlen, one
 *     row per packed sequence); bias_ij = -slope(b, h) * |c_i - j|, added after the
 *     scaling.  alibi_per_batch must be 0 or 1 (it is ignored without slopes).
 *   - A row with no visible key gets out = 0 and lse = -inf.
 *   - softmax_scale is used exactly as given (any finite value, negative included).
 *   - headdim must be 64, 128 or 256.
 *
 * Ownership and streams
 *   - All pointers except the return value of fa_status_str are DEVICE pointers owned
 *     by the caller.  The library allocates nothing, keeps no mutable global state
 *     (calls from several host threads are safe) and never synchronises.
 *   - Work is enqueued on `stream` (0 = the default stream); a call returns after
 *     the enqueue.  Buffers must stay valid until the work has run.
 *   - Inputs are read only.  Output buffers must not alias the inputs.
 *
 * Errors (return value)
 *   FA_OK (0) on success.  On any error nothing is launched and no output is touched:
 *   FA_ERR_INVALID_ARG (-1): a NULL required pointer, a 16-bit tensor pointer that is
 *                            not 16-byte aligned, a size < 1, a window side < -1,
 *                            num_splits outside [1, seqlen_k], a non-finite softmax_scale,
 *                            a dtype other than FA_BF16 / FA_FP16, alibi_per_batch
 *                            other than 0 / 1, a problem whose element count
 *                            overflows 64-bit indexing, or a call one of whose
 *                            kernel grids would exceed the runtime's 2^32 - 1
 *                            work-items (2^24 - 1 workgroups of 256 threads; the
 *                            eight-wave headdim-128 forward 2^23 - 1 of 512); every
 *                            grid of a call is checked before its first launch;
 *   FA_ERR_UNSUPPORTED (-2): headdim not in {64, 128, 256}, or nheads * headdim > 2^22;
 *   FA_ERR_LAUNCH      (-3): the HIP runtime reported an error for the launch.
 *   No exception crosses the ABI and nothing is printed.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK 0
#define FA_ERR_INVALID_ARG (-1)
#define FA_ERR_UNSUPPORTED (-2)
#define FA_ERR_LAUNCH (-3)

/* element type of the 16-bit tensors (the dtype argument) */
#define FA_BF16 0
#define FA_FP16 1

/*
 * fa_fwd - attention forward for a padded batch [FA-overview, "使用示例", "参数说明",
 * "算法 / 前向传播", "2.1", "2.3"].
 *   q      [batch, seqlen_q, nheads, headdim] dtype (device, read)
 *   k, v   [batch, seqlen_k, nheads, headdim] dtype (device, read)
 *   out    [batch, seqlen_q, nheads, headdim] dtype (device, written)
 *   lse    [batch, nheads, seqlen_q]          fp32 (device, written)
 *   causal, window_left, window_right, alibi_slopes, alibi_per_batch, dtype: see the
 *   conventions above.
 * One workgroup per (batch, head, block of 128 query rows); every output element
 * is written exactly once, without atomics, so results are bitwise reproducible.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
           int batch, int seqlen_q, int seqlen_k, int nheads, int headdim,
           float softmax_scale, int causal, int window_left, int window_right,
           const float* alibi_slopes, int alibi_per_batch, int dtype, hipStream_t stream);

/*
 * fa_fwd_splitkv - first half of the split-KV forward [FA-overview, "2.2"].
 * The keys are cut into num_splits contiguous ranges: split s covers
 * [s*C, min(seqlen_k, (s+1)*C)) with C = ceil(seqlen_k / num_splits).  For each
 * split it writes the attention restricted to that split's visible keys:
 *   out_partial [num_splits, batch, nheads, seqlen_q, headdim] fp32 (device, written),
 *               normalised within the split (0 where the split sees no key);
 *   lse_partial [num_splits, batch, nheads, seqlen_q] fp32 (device, written),
 *               -inf where the split sees no key.
 * The other arguments mean what they mean for fa_fwd.  Follow with fa_combine on
 * the same stream.  Rows of short queries (seqlen_q <= 8) run on a vector-ALU
 * kernel that streams the KV cache; longer queries run on the matrix-core kernel.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v,
                   float* out_partial, float* lse_partial,
                   int batch, int seqlen_q, int seqlen_k, int nheads, int headdim,
                   float softmax_scale, int causal, int window_left, int window_right,
                   const float* alibi_slopes, int alibi_per_batch, int dtype, int num_splits,
                   hipStream_t stream);

/*
 * fa_fwd_varlen - attention forward over a packed batch of sequences of different
 * lengths, with grouped K/V heads [FA-overview, "函数重命名" (the variable-length
 * interface), "代码解读：FlashSelfAttention" (packed rows indexed by cu_seqlens),
 * "代码解读博客：FlashCrossAttention" (separate cu_seqlens_k / max_seqlen_k, K/V
 * with their own head count H_k)].
 *   cu_seqlens_q [batch + 1] int32 (device, read): sequence b owns q/out rows
 *                [cu_seqlens_q[b], cu_seqlens_q[b+1]); cu_seqlens_q[0] = 0 and the
 *                array is non-decreasing;
 *   cu_seqlens_k [batch + 1] int32 (device, read): the same for k/v rows;
 *   q, out [total_q, nheads, headdim]   dtype (device), total_q = cu_seqlens_q[batch]
 *   k, v   [total_k, nheads_k, headdim] dtype (device), total_k = cu_seqlens_k[batch]
 *   lse    [nheads, total_q]            fp32 (device, written)
 *   max_seqlen_q, max_seqlen_k: at least every sequence's length (they size the grid;
 *                rows of a longer sequence past max_seqlen_q are left unwritten);
 *   nheads_k: divides nheads; query head h reads K/V head h / (nheads / nheads_k)
 *             (nheads_k = nheads: ordinary multi-head, 1: a single shared K/V head).
 * Each sequence is its own attention problem: causal alignment, windows and ALiBi
 * use that sequence's lengths (query i of sequence b sits at key position
 * i + Sk_b - Sq_b).  alibi_slopes is indexed by query head (and by sequence when
 * alibi_per_batch is 1).  The cu_seqlens arrays
 * are read on the device only, so the host cannot check them: they must describe
 * rows inside q/k/v/out (an invalid array makes the kernel read or write outside
 * the buffers).  Errors as for fa_fwd, plus FA_ERR_INVALID_ARG for a NULL cu_seqlens
 * pointer, total_q < 1, nheads_k < 1 or nheads_k not dividing nheads.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int max_seqlen_q,
                  int max_seqlen_k, int total_q, int nheads, int nheads_k, int headdim,
                  float softmax_scale, int causal, int window_left, int window_right,
                  const float* alibi_slopes, int alibi_per_batch, int dtype, hipStream_t stream);

/*
 * fa_combine - second half of the split-KV forward [FA-overview, "2.2"].
 * Per row: L = ln sum_s exp(lse_partial[s]); out = sum_s exp(lse_partial[s] - L) *
 * out_partial[s]; lse = L.  A row where every split is empty gets out = 0, lse = -inf.
 *   out_partial, lse_partial: as written by fa_fwd_splitkv (device, read)
 *   out [batch, seqlen_q, nheads, headdim] dtype (device, written)
 *   lse [batch, nheads, seqlen_q]          fp32 (device, written)
 * num_splits must be >= 1 (the partial layout does not depend on seqlen_k).
 */
int fa_combine(const float* out_partial, const float* lse_partial, void* out, float* lse,
               int batch, int seqlen_q, int nheads, int headdim, int num_splits, int dtype,
               hipStream_t stream);

/*
 * fa_fwd_kvcache - decode step against a KV cache [FA-overview, "2.2" (short queries:
 * the keys are split across workgroups and merged by a second kernel; the KV-cache
 * entry rotates q and the new keys and appends them to the cache in place), "2.5"
 * (paged KV cache)].
 *   q [batch, seqlen_q, nheads, headdim] dtype (device, read), 1 <= seqlen_q <= 8
 *   k_cache, v_cache (device, read and written): block_table != NULL: paged,
 *       [num_blocks, page_size, nheads_k, headdim] dtype, logical block n of sequence b
 *       is physical block block_table[b * max_blocks_per_seq + n]; page_size a power of
 *       two, at least 64;  block_table == NULL: contiguous [batch, page_size, nheads_k,
 *       headdim], page_size being the capacity per sequence.
 *   cache_seqlens [batch] int32 (device, read): rows already in the cache.
 *   k_new, v_new [batch, seqlen_new, nheads_k, headdim] dtype (device, read) or NULL when
 *       seqlen_new = 0: appended at rows cache_seqlens[b] .. + seqlen_new - 1 (written into
 *       the cache before the attention reads it).
 *   rotary_cos, rotary_sin [positions, rotary_dim / 2] fp32 (device, read) or both NULL,
 *       with a row for every cache position (positions >= the capacity: page_size *
 *       max_blocks_per_seq, or page_size for a contiguous cache):
 *       query row i and new key row i are rotated at position cache_seqlens[b] + i, pairs
 *       (x_d, x_{d + rotary_dim/2}) for d < rotary_dim / 2 (rotary_dim even, <= headdim);
 *       the rotated keys are stored in the cache, rounded to dtype.
 *   out [batch, seqlen_q, nheads, headdim] dtype, lse [batch, nheads, seqlen_q] fp32
 *       (device, written; out also holds the rotated queries between the two passes).
 *   out_partial, lse_partial: caller-owned scratch of at least max_splits splits in the
 *       fa_fwd_splitkv layout.  num_splits = 0 picks the split count (about 2048
 *       workgroups when a workgroup serves one or two queries of a K/V head, about 512
 *       when it serves four or eight; at least 256 keys per split), else 1..max_splits.
 * Sequence b attends to its cache_seqlens[b] + seqlen_new keys; the causal/window
 * alignment is bottom-right within them.  Query head h reads K/V head
 * h / (nheads / nheads_k).  Device-side values (cache_seqlens, block_table, rotary
 * positions) cannot be checked on the host: they must stay inside the buffers.
 * Errors as for fa_fwd, plus FA_ERR_INVALID_ARG for NULL required pointers, seqlen_q
 * outside [1, 8], an invalid page_size, rotary_dim, num_splits or head grouping, or
 * seqlen_new larger than the capacity.
 */
int fa_fwd_kvcache(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens,
                   const int* block_table, int page_size, int max_blocks_per_seq,
                   const void* k_new, const void* v_new, int seqlen_new,
                   const float* rotary_cos, const float* rotary_sin, int rotary_dim,
                   void* out, float* lse, float* out_partial, float* lse_partial, int max_splits,
                   int batch, int seqlen_q, int nheads, int nheads_k, int headdim,
                   float softmax_scale, int causal, int window_left, int window_right,
                   const float* alibi_slopes, int alibi_per_batch, int dtype, int num_splits,
                   hipStream_t stream);

/*
 * fa_bwd - gradients of the attention forward [FA-overview, "算法 / 反向传播": P is
 * recomputed from the row-wise logsumexp L alone; "并行性 / 反向传播": one block per
 * K/V column block].  With S = softmax_scale * Q K^T + bias on the visible pairs and
 * P = exp(S - L):
 *   dV = P^T dO,  D = rowsum(dO o O),  dS = P o (dO V^T - D),
 *   dQ = softmax_scale * dS K,  dK = softmax_scale * dS^T Q.
 *   q, k, v, out   as for fa_fwd; out and lse are the forward's outputs (device, read)
 *   dout [batch, seqlen_q, nheads, headdim] dtype (device, read): gradient of out
 *   dq   [batch, seqlen_q, nheads, headdim] dtype (device, written)
 *   dk, dv [batch, seqlen_k, nheads, headdim] dtype (device, written)
 *   delta [batch, nheads, seqlen_q] fp32 (device): caller-owned scratch, written with D
 *   The other arguments mean what they mean for fa_fwd and must be the forward's.
 * Rows with no visible key (lse = -inf) get dq = 0 and add nothing to dk, dv.  Keys no
 * query sees get dk = dv = 0.  Every output element is written exactly once (no
 * atomics): results are bitwise reproducible.  The ALiBi slopes are constants here
 * (no gradient).  headdim 64, 128 or 256.  Errors as for
 * fa_fwd, plus FA_ERR_INVALID_ARG for a NULL out, lse, dout, dq, dk, dv or delta.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta,
           int batch, int seqlen_q, int seqlen_k, int nheads, int headdim,
           float softmax_scale, int causal, int window_left, int window_right,
           const float* alibi_slopes, int alibi_per_batch, int dtype, hipStream_t stream);

/*
 * fa_bwd_varlen - gradients of fa_fwd_varlen: the backward of fa_bwd over a packed
 * batch of sequences with grouped K/V heads [FA-overview, "算法 / 反向传播",
 * "并行性 / 反向传播"; the packed layout and the K/V head groups as for fa_fwd_varlen
 * ("代码解读：FlashSelfAttention", "代码解读博客：FlashCrossAttention")].
 *   q, out, dout, dq [total_q, nheads, headdim]   dtype (device; dq written)
 *   k, v, dk, dv     [total_k, nheads_k, headdim] dtype (device; dk, dv written)
 *   lse              [nheads, total_q] fp32 (device, read): fa_fwd_varlen's output
 *   delta            [nheads, total_q] fp32 (device): caller-owned scratch, written with D
 *   cu_seqlens_q/k, batch, max_seqlen_q/k, nheads_k and the mask arguments as for
 *   fa_fwd_varlen (and the forward's values); total_k = cu_seqlens_k[batch].
 * A K/V head's dk and dv sum the contributions of every query head of its group
 * (the forward reads it once per query head); the sums are formed in one workgroup,
 * in a fixed order, so results are bitwise reproducible.  Rows of a sequence past
 * max_seqlen_q (or keys past max_seqlen_k) are left unwritten; the cu_seqlens arrays
 * are read on the device only and must describe rows inside the tensors.  headdim
 * 64, 128 or 256.  Errors as for fa_bwd, plus FA_ERR_INVALID_ARG for a NULL
 * cu_seqlens pointer, total_q < 1, total_k < 1, nheads_k < 1 or nheads_k not dividing
 * nheads.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, float* delta,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int max_seqlen_q,
                  int max_seqlen_k, int total_q, int total_k, int nheads, int nheads_k, int headdim,
                  float softmax_scale, int causal, int window_left, int window_right,
                  const float* alibi_slopes, int alibi_per_batch, int dtype, hipStream_t stream);

/*
 * fa_fwd_kvcache_noalloc - fa_fwd_kvcache for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, kernels and results, without out_partial,
 * lse_partial and max_splits.  The split partials live in a device buffer the
 * library holds, 16 MiB per GPU (FA_NOALLOC_SCRATCH_BYTES), for the life of the
 * process; the call itself allocates nothing.  At most
 *     floor(16 MiB / (batch * nheads * seqlen_q * (4 * headdim + 4)))
 * splits fit (e.g. 254 for batch 8, 16 heads, one query row, headdim 128):
 * num_splits = 0 caps the automatic count there, a larger explicit num_splits, or a
 * step whose single split does not fit, returns FA_ERR_INVALID_ARG.  The buffer of a
 * GPU is looked up on the first call that runs there (on the device of `stream`).
 * All calls on one GPU share it: calls that overlap in time on one GPU (on two
 * streams, or from two host threads) race, and must be ordered by the caller.
 * FA_ERR_LAUNCH also reports a failed lookup of the buffer.
 */
int fa_fwd_kvcache_noalloc(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens,
                           const int* block_table, int page_size, int max_blocks_per_seq,
                           const void* k_new, const void* v_new, int seqlen_new,
                           const float* rotary_cos, const float* rotary_sin, int rotary_dim,
                           void* out, float* lse,
                           int batch, int seqlen_q, int nheads, int nheads_k, int headdim,
                           float softmax_scale, int causal, int window_left, int window_right,
                           const float* alibi_slopes, int alibi_per_batch, int dtype, int num_splits,
                           hipStream_t stream);

/* fa_status_str - static, human-readable name of a status code (never NULL). */
const char* fa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
