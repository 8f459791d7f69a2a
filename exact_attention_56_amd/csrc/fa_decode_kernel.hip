// fa_decode_kernel.hip - split-KV decode partial kernel, KV-cache preparation and the
// combine kernel (gfx950).
//
// Page "FlashAttention：快速且内存高效的准确注意力机制"
// (cloud.tencent.com.cn/developer/article/2433927), section "2.2：针对推理进行优化":
// with very short queries the cost is reading the KV cache, so the keys are split
// across workgroups and a separate kernel merges the per-split results; section
// "2.5" (paged KV cache) for the block-table reads.
//
// Partial kernel: a few query rows against a KV chunk are matrix-vector products,
// so they run on the vector ALUs and are bound by HBM bandwidth.  One workgroup per
// (batch, K/V head, split, chunk of up to eight queries of that K/V head); each key
// row (headdim 16-bit values) is read by HD/8 lanes with one 16-byte load each, and
// the four waves walk interleaved slices of the chunk with their own online-softmax
// state, merged through LDS at the end.  The output of a split is normalised within
// the split, with its logsumexp; an empty split gives 0 and -inf.
//
// Combine kernel: out = sum_s exp(lse_s - L) out_s with L = ln sum_s exp(lse_s), one
// workgroup per row.
#include "fa_fwd_kernel.h"  // decode_uses_mfma, launch_fwd_decode_d64/d128 (compiled with their own flags)

namespace fa {

constexpr int DEC_THREADS = BLOCK_THREADS;
#ifndef FA_DEC_CPOL
#define FA_DEC_CPOL 2
#endif
constexpr int DEC_CPOL = FA_DEC_CPOL;      // KV loads are non-temporal (read once, streamed)

// Helpers of the grouped kernel.  Dot product of 8 packed 16-bit values (two 16-byte
// chunks) in fp32: four v_dot2 instructions.  Each element is copied to a scalar
// before the bit cast: a bit cast applied directly to a vector element expression
// was compiled as a cast of element 0 every time.
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float acc, __bf16) {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t ae = a[e], be = b[e];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, ae), __builtin_bit_cast(v2, be), acc, false);
  }
  return acc;
}
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float acc, _Float16) {
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t ae = a[e], be = b[e];
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, ae), __builtin_bit_cast(v2, be), acc, false);
  }
  return acc;
}

// x of lane (l op CTRL) within its 16-lane row (DPP; every lane has a source).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the LPR consecutive lanes (8, 16 or 32) that share a key row, returned in
// all of them: two quad permutations, then within 8 lanes the half-row mirror, or
// within 16 the row rotations by 4 and 8; 32 adds one swap of the 16-lane halves.
template <int LPR>
__device__ __forceinline__ float lane_group_sum(float x) {
  x += dpp_move<0xB1>(x);  // quad_perm [1, 0, 3, 2]
  x += dpp_move<0x4E>(x);  // quad_perm [2, 3, 0, 1]
  if constexpr (LPR == 8) x += dpp_move<0x141>(x);  // row_half_mirror: the other quad
  if constexpr (LPR >= 16) {
    x += dpp_move<0x124>(x);  // row_ror 4
    x += dpp_move<0x128>(x);  // row_ror 8
  }
  if constexpr (LPR == 32) x += __shfl_xor(x, 16);
  return x;
}

// Decode partial kernel: one workgroup per (batch, K/V head, split, chunk of NQ
// queries).  The queries of a K/V head are its nheads / nheads_k query heads times
// the seqlen_q rows (query n: head hk * G + n / Sq, row n % Sq); one workgroup takes NQ
// of them, so each key row it loads serves NQ dot products.  Each query keeps its own
// visible range and ALiBi slope.
//
// HD/8 lanes per key row (one 16-byte chunk each), 64/(HD/8) rows per wave per load.
// The dot products take packed v_dot2 instructions on the raw 16-bit values, the
// lane-group sums run on DPP moves (no LDS permutes), every row group of a wave
// keeps its own online-softmax state (merged once at the end, so no per-step
// exchange of maxima), the reference maximum moves only when a score exceeds it by
// more than 2^8 (as in the forward kernel), and steps inside every query's visible
// range skip the mask.
//
// KVC: the keys come from a KV cache (fa_fwd_kvcache): sequence b has
// cache_seqlens[b] + seqlen_new keys, and block n of it lives in block
// block_table[b, n] (or block b of a contiguous cache).  Steps then start on
// multiples of STEP so that none crosses a block; keys below the range are masked.
template <int HD, bool ALIBI, bool KVC, int NQ, typename E>
__global__ __launch_bounds__(DEC_THREADS) void decode_group_kernel(FwdParams p) {
  constexpr int LPR = HD / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int UNROLL = NQ <= 2 ? DEC_UNROLL : DEC_UNROLL / 2;  // registers: NQ copies of the state
  constexpr int STEP = UNROLL * RPW;
  constexpr float TH = 8.0f;  // log2 units: keep a stale reference maximum while p <= 2^8
  __shared__ float sm_m[4][NQ], sm_l[4][NQ];
  __shared__ float sm_acc[4][NQ][HD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane / LPR;
  const int cidx = lane % LPR;

  const int Sq = p.seqlen_q;
  const int G = p.nheads / p.nheads_k;
  const int nq_total = G * Sq;
  const int nchunks = (nq_total + NQ - 1) / NQ;
  int w = xcd_remap(blockIdx.x, gridDim.x);
  const int qc = w % nchunks;
  w /= nchunks;
  const int split = w % p.num_splits;
  w /= p.num_splits;
  const int hk = w % p.nheads_k;
  const int b = w / p.nheads_k;
  const int Sk = KVC ? p.cache_seqlens[b] + p.seqlen_new : p.seqlen_k;

  const long row_stride = (long)p.nheads * HD;
  const long kv_stride = (long)p.nheads_k * HD;
  const int row_bytes = (int)kv_stride * 2;
  const int s_lo = min(Sk, split * p.split_len);
  const int s_hi = min(Sk, s_lo + p.split_len);

  const float c = (p.q_sign ? -p.scale_log2 : p.scale_log2);
  u32x4 qv[NQ];
  float slope[NQ];
  int q_lo[NQ], q_hi[NQ], q_pos[NQ];
  int lo = s_hi, hi = s_lo;              // union of the queries' visible ranges in this split
  int in_lo = s_lo, in_hi = s_hi;        // keys every query of the chunk sees
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int n = qc * NQ + j;
    const bool valid = n < nq_total;
    const int h = hk * G + (valid ? n / Sq : 0);
    const int i = valid ? n % Sq : 0;
    q_pos[j] = i + Sk - Sq;
    int l0 = s_lo, h0 = s_hi;
    if (p.window_left >= 0) l0 = max(l0, q_pos[j] - p.window_left);
    if (p.window_right >= 0) h0 = min(h0, q_pos[j] + p.window_right + 1);
    if (!valid) h0 = l0;  // an empty query
    q_lo[j] = l0;
    q_hi[j] = h0;
    if (h0 > l0) {
      lo = min(lo, l0);
      hi = max(hi, h0);
    }
    if (valid) {
      in_lo = max(in_lo, l0);
      in_hi = min(in_hi, h0);
    }
    qv[j] = valid ? *(const u32x4*)(p.q + ((long)b * Sq + i) * row_stride + (long)h * HD + cidx * 8) & p.q_and
                  : u32x4{0u, 0u, 0u, 0u};
    slope[j] = 0.f;
    if constexpr (ALIBI) slope[j] = p.alibi[(long)b * p.alibi_bstride + h] * kLog2e;
  }
  if (hi <= lo) lo = hi = 0;  // no query sees a key of this split
  const long kvb = KVC ? (long)hk * HD : (long)b * Sk * kv_stride + (long)hk * HD;
  const int first = KVC ? (lo & ~(STEP - 1)) : lo;

  float m_run[NQ], l_run[NQ], acc[NQ][8];  // per row group of the wave
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }

  for (int base = first + wave * STEP; base < hi; base += 4 * STEP) {
    const int nrec = min(hi - base, STEP) * row_bytes;
    long row0 = base;
    if constexpr (KVC) {
      if (p.block_table != nullptr)
        row0 = (long)p.block_table[(long)b * p.max_blocks + (base >> p.page_shift)] * p.page_size +
               (base & (p.page_size - 1));
      else
        row0 = (long)b * p.page_size + base;
    }
    const auto krs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kvb + row0 * kv_stride), (short)0, nrec,
                                                       0x00020000);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kvb + row0 * kv_stride), (short)0, nrec,
                                                       0x00020000);
    u32x4 kr[UNROLL], vr[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int off = (u * RPW + g) * row_bytes + cidx * 16;
      kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, DEC_CPOL));
      vr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, DEC_CPOL));
    }
    const bool inside = base >= in_lo && base + STEP <= in_hi;  // wave-uniform
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float sj[UNROLL];
      float bmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float part = lane_group_sum<LPR>(dot8(qv[j], kr[u], 0.f, E{})) * c;
        const int key = base + u * RPW + g;
        if constexpr (ALIBI) part -= slope[j] * fabsf((float)(q_pos[j] - key));
        sj[u] = (inside || (key >= q_lo[j] && key < q_hi[j])) ? part : -INFINITY;
        bmax = fmaxf(bmax, sj[u]);
      }
      const bool grow = bmax > m_run[j] + TH;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = !grow ? 1.f : (m_run[j] == -INFINITY ? 0.f : fast_exp2(m_run[j] - bmax));
        m_run[j] = grow ? bmax : m_run[j];
        l_run[j] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] *= alpha;
      }
      // a group whose reference is still -inf has seen only masked keys: p = 0
      const float m_use = (m_run[j] == -INFINITY) ? 0.f : m_run[j];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const float pu = fast_exp2(sj[u] - m_use);
        l_run[j] += pu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[j][2 * e] = fmaf(pu, widen_lo<E>(vr[u][e]), acc[j][2 * e]);
          acc[j][2 * e + 1] = fmaf(pu, widen_hi<E>(vr[u][e]), acc[j][2 * e + 1]);
        }
      }
    }
  }

  // merge the row groups of each wave (each against its own reference), then the
  // four waves, per query
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    float M = m_run[j];
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float sc = (m_run[j] == -INFINITY) ? 0.f : fast_exp2(m_run[j] - M);
    l_run[j] *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] *= sc;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      l_run[j] += __shfl_xor(l_run[j], o);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] += __shfl_xor(acc[j][e], o);
    }
    if (lane == 0) {
      sm_m[wave][j] = M;
      sm_l[wave][j] = l_run[j];
    }
    if (g == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][j][cidx * 8 + e] = acc[j][e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int n = qc * NQ + j;
    if (n >= nq_total) break;
    const int h = hk * G + n / Sq, i = n % Sq;
    const float M = fmaxf(fmaxf(sm_m[0][j], sm_m[1][j]), fmaxf(sm_m[2][j], sm_m[3][j]));
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float wgt[4], L = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      wgt[x] = fast_exp2(sm_m[x][j] - M_use);
      L += sm_l[x][j] * wgt[x];
    }
    const long rowid = (((long)split * p.batch + b) * p.nheads + h) * Sq + i;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float* out = (float*)p.out + rowid * HD;
    for (int d = tid; d < HD; d += DEC_THREADS) {
      float o = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) o = fmaf(sm_acc[x][j][d], wgt[x], o);
      out[d] = o * inv;
    }
    if (tid == 0) p.lse[rowid] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
  }
}

// Maximum / sum of x over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// One workgroup per output row.  The reads of a row's partials are issued before
// anything waits: each thread loads up to CPB partial chunks (16 bytes of one split's
// row; HD/4 threads cover a row, 256/(HD/4) splits side by side), and every wave
// reads the splits' lse values itself and reduces them (maximum, then the sum of
// the weights exp(lse_s - max)) with lane exchanges, so the weights need no barrier.
// The split groups are added through LDS at the end.  A split whose lse is -inf
// (no visible key) gets weight 0 and its partial row is ignored, whatever it holds.
template <int HD, typename E>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int TPS = HD / 4;     // threads per partial row (4 floats each)
  constexpr int SPP = 256 / TPS;  // partial rows side by side
  constexpr int CPB = 8;          // partial chunks in flight per thread
  __shared__ __attribute__((aligned(16))) float sm_acc[SPP][HD];
  const int tid = threadIdx.x, lane = tid & 63;
  const long rows = (long)p.batch * p.nheads * p.seqlen_q;
  const long row = blockIdx.x;  // (b*H + h)*Sq + i
  const int i = (int)(row % p.seqlen_q);
  const long bh = row / p.seqlen_q;
  const int h = (int)(bh % p.nheads);
  const int b = (int)(bh / p.nheads);
  const int ns = p.num_splits;
  const float* lp = p.lse_partial + row;
  const float* op = p.out_partial + row * HD;
  const long lstride = rows, ostride = rows * HD;
  const int sg = tid / TPS, c = tid % TPS;

  f32x4 v[CPB];
#pragma unroll
  for (int k = 0; k < CPB; ++k) {
    const int s = sg + SPP * k;
    v[k] = s < ns ? *(const f32x4*)(op + s * ostride + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, lp[s * lstride]);
  const float M = wave_max(mx);
  const float M_use = (M == -INFINITY) ? 0.f : M;
  float sum = 0.f;
  for (int s = lane; s < ns; s += 64) sum += fast_exp2((lp[s * lstride] - M_use) * kLog2e);  // 0: empty split
  const float L = wave_sum(sum);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0;; s0 += SPP * CPB) {
#pragma unroll
    for (int k = 0; k < CPB; ++k) {
      const int s = s0 + sg + SPP * k;
      if (s < ns) {
        const float wgt = fast_exp2((lp[s * lstride] - M_use) * kLog2e);
        if (wgt != 0.f) acc += wgt * v[k];
      }
    }
    if (s0 + SPP * CPB >= ns) break;
#pragma unroll
    for (int k = 0; k < CPB; ++k) {
      const int s = s0 + SPP * CPB + sg + SPP * k;
      v[k] = s < ns ? *(const f32x4*)(op + s * ostride + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  *(f32x4*)&sm_acc[sg][4 * c] = acc;
  __syncthreads();
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* out = p.out + (((long)b * p.seqlen_q + i) * p.nheads + h) * HD;
  if (tid < HD) {
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < SPP; ++g) o += sm_acc[g][tid];
    out[tid] = (uint16_t)(pack2<E>(o * inv, 0.f) & 0xffffu);
  }
  if (tid == 0) p.lse[row] = L > 0.f ? M + logf(L) : -INFINITY;
}

// Element e of a row x of E rotated at position `pos` (half-split rotary layout:
// the pair (x_d, x_{d + rd/2}) turns by the angle of cos[pos, d], sin[pos, d];
// columns from rd on are unchanged), rounded to E.
template <typename E>
__device__ __forceinline__ uint16_t rotated(const uint16_t* x, int e, long pos, const float* cos, const float* sin,
                                            int rd) {
  const int half = rd >> 1;
  const float xe = widen_lo<E>(x[e]);
  float y = xe;
  if (e < half) {
    const float c = cos[pos * half + e], s = sin[pos * half + e];
    y = xe * c - widen_lo<E>(x[e + half]) * s;
  } else if (e < rd) {
    const float c = cos[pos * half + e - half], s = sin[pos * half + e - half];
    y = xe * c + widen_lo<E>(x[e - half]) * s;
  }
  return (uint16_t)(pack2<E>(y, 0.f) & 0xffffu);
}

// KV-cache preparation, one wave per row: rows [0, n_kv) append k_new / v_new row
// (b, i, hk) at position cache_seqlens[b] + i of the cache (keys rotated when cos is
// given); rows [n_kv, n_kv + n_q) write query row (b, i, h) rotated at position
// cache_seqlens[b] + i into qrot.
template <int HD, typename E>
__global__ __launch_bounds__(256) void kvcache_prep_kernel(FwdParams p, const uint16_t* k_new, const uint16_t* v_new,
                                                           uint16_t* k_cache, uint16_t* v_cache, const float* cos,
                                                           const float* sin, int rd, uint16_t* qrot, long n_kv,
                                                           long n_q) {
  const int lane = threadIdx.x & 63;
  const long task = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task < n_kv) {
    const int hk = (int)(task % p.nheads_k);
    const long bi = task / p.nheads_k;
    const int i = (int)(bi % p.seqlen_new);
    const int b = (int)(bi / p.seqlen_new);
    const int j = p.cache_seqlens[b] + i;
    const long row = p.block_table != nullptr
                         ? (long)p.block_table[(long)b * p.max_blocks + (j >> p.page_shift)] * p.page_size +
                               (j & (p.page_size - 1))
                         : (long)b * p.page_size + j;
    const long src = bi * p.nheads_k * HD + (long)hk * HD;
    const long dst = (row * p.nheads_k + hk) * HD;
    for (int e = lane; e < HD; e += 64) {
      k_cache[dst + e] = cos != nullptr ? rotated<E>(k_new + src, e, j, cos, sin, rd) : k_new[src + e];
      v_cache[dst + e] = v_new[src + e];
    }
  } else if (task < n_kv + n_q) {
    const long t = task - n_kv;  // ((b * Sq) + i) * H + h
    const long bi = t / p.nheads;
    const int i = (int)(bi % p.seqlen_q);
    const int b = (int)(bi / p.seqlen_q);
    const long pos = (long)p.cache_seqlens[b] + i;
    for (int e = lane; e < HD; e += 64) qrot[t * HD + e] = rotated<E>(p.q + t * HD, e, pos, cos, sin, rd);
  }
}

template <int HD, bool ALIBI, bool KVC, int NQ, typename E>
static void launch_group(const FwdParams& p, hipStream_t stream) {
  const int nq_total = p.nheads / p.nheads_k * p.seqlen_q;
  const long nblocks = (long)p.batch * p.nheads_k * p.num_splits * ((nq_total + NQ - 1) / NQ);
  hipLaunchKernelGGL((decode_group_kernel<HD, ALIBI, KVC, NQ, E>), dim3((unsigned)nblocks), dim3(DEC_THREADS), 0,
                     stream, p);
}

template <int HD, bool ALIBI, bool KVC, typename E>
static void launch_group_nq(const FwdParams& p, hipStream_t stream) {
  switch (decode_queries_per_block(p.nheads / p.nheads_k * p.seqlen_q)) {
    case 1: launch_group<HD, ALIBI, KVC, 1, E>(p, stream); break;
    case 2: launch_group<HD, ALIBI, KVC, 2, E>(p, stream); break;
    case 4: launch_group<HD, ALIBI, KVC, 4, E>(p, stream); break;
    default: launch_group<HD, ALIBI, KVC, 8, E>(p, stream); break;
  }
}

template <int HD, bool KVC, typename E>
static hipError_t launch_decode_kvc(const FwdParams& p, hipStream_t stream) {
  if (p.alibi) launch_group_nq<HD, true, KVC, E>(p, stream);
  else launch_group_nq<HD, false, KVC, E>(p, stream);
  return hipGetLastError();
}

template <int HD, typename E>
static hipError_t launch_kvcache_hd(const FwdParams& p, const uint16_t* k_new, const uint16_t* v_new,
                                    uint16_t* k_cache, uint16_t* v_cache, const float* cos, const float* sin, int rd,
                                    uint16_t* qrot, hipStream_t stream) {
  const long n_kv = (long)p.batch * p.seqlen_new * p.nheads_k;
  const long n_q = cos != nullptr ? (long)p.batch * p.seqlen_q * p.nheads : 0;
  if (n_kv + n_q > 0)
    hipLaunchKernelGGL((kvcache_prep_kernel<HD, E>), dim3((unsigned)((n_kv + n_q + 3) / 4)), dim3(256), 0, stream,
                       p, k_new, v_new, k_cache, v_cache, cos, sin, rd, qrot, n_kv, n_q);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FwdParams d = p;
  if (cos != nullptr) d.q = qrot;  // the decode kernel reads the rotated queries
  if constexpr (HD != 256) {
    // more than four queries per K/V head: every K/V tile feeds matrix-core products for
    // all of them (the vector-ALU kernel's work per key grows with their number)
    if (decode_uses_mfma(HD, p.nheads / p.nheads_k * p.seqlen_q)) {
      d.split_len = (p.split_len + BC - 1) / BC * BC;
      return HD == 64 ? launch_fwd_decode_d64(d, stream) : launch_fwd_decode_d128(d, stream);
    }
  }
  return launch_decode_kvc<HD, true, E>(d, stream);
}

template <typename E>
static hipError_t launch_kvcache_e(const FwdParams& p, int headdim, const uint16_t* k_new, const uint16_t* v_new,
                                   uint16_t* k_cache, uint16_t* v_cache, const float* cos, const float* sin, int rd,
                                   uint16_t* qrot, hipStream_t stream) {
  switch (headdim) {
    case 64: return launch_kvcache_hd<64, E>(p, k_new, v_new, k_cache, v_cache, cos, sin, rd, qrot, stream);
    case 128: return launch_kvcache_hd<128, E>(p, k_new, v_new, k_cache, v_cache, cos, sin, rd, qrot, stream);
    case 256: return launch_kvcache_hd<256, E>(p, k_new, v_new, k_cache, v_cache, cos, sin, rd, qrot, stream);
    default: return hipErrorInvalidValue;
  }
}

// KV-cache decode: append (and rotate), then the split partials.  The caller runs
// the combine afterwards.
hipError_t launch_kvcache(const FwdParams& p, int headdim, const uint16_t* k_new, const uint16_t* v_new,
                          uint16_t* k_cache, uint16_t* v_cache, const float* cos, const float* sin, int rd,
                          uint16_t* qrot, hipStream_t stream) {
  return p.f16 ? launch_kvcache_e<_Float16>(p, headdim, k_new, v_new, k_cache, v_cache, cos, sin, rd, qrot, stream)
               : launch_kvcache_e<__bf16>(p, headdim, k_new, v_new, k_cache, v_cache, cos, sin, rd, qrot, stream);
}

template <typename E>
static hipError_t launch_decode_e(const FwdParams& p, int headdim, hipStream_t stream) {
  switch (headdim) {
    case 64: return launch_decode_kvc<64, false, E>(p, stream);
    case 128: return launch_decode_kvc<128, false, E>(p, stream);
    case 256: return launch_decode_kvc<256, false, E>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const FwdParams& p, int headdim, hipStream_t stream) {
  return p.f16 ? launch_decode_e<_Float16>(p, headdim, stream) : launch_decode_e<__bf16>(p, headdim, stream);
}

template <typename E>
static hipError_t launch_combine_e(const CombineParams& p, int headdim, hipStream_t stream) {
  const long rows = (long)p.batch * p.nheads * p.seqlen_q;
  const dim3 grid((unsigned)rows);
  switch (headdim) {
    case 64: hipLaunchKernelGGL((combine_kernel<64, E>), grid, dim3(256), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((combine_kernel<128, E>), grid, dim3(256), 0, stream, p); break;
    case 256: hipLaunchKernelGGL((combine_kernel<256, E>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int headdim, hipStream_t stream) {
  return p.f16 ? launch_combine_e<_Float16>(p, headdim, stream) : launch_combine_e<__bf16>(p, headdim, stream);
}

}  // namespace fa
