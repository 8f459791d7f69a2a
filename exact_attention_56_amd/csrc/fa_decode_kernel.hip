// fa_decode_kernel.hip - split-KV decode partial kernel and the combine kernel (gfx950).
//
// Page "FlashAttention：快速且内存高效的准确注意力机制"
// (cloud.tencent.com.cn/developer/article/2433927), section "2.2：针对推理进行优化":
// with very short queries the cost is reading the KV cache, so the keys are split
// across workgroups and a separate kernel merges the per-split results.
//
// Partial kernel: one workgroup per (batch, head, split, query row).  A query row
// against a KV chunk is a matrix-vector product, so it runs on the vector ALUs and
// is bound by HBM bandwidth: each key row (headdim 16-bit values) is read by HD/8 lanes with
// one 16-byte load each, the dot product is finished with lane shuffles, and the
// four waves walk interleaved slices of the chunk with their own online-softmax
// state, merged through LDS at the end.  The output of a split is normalised
// within the split, with its logsumexp; an empty split gives 0 and -inf.
// When a K/V head serves several queries (grouped heads, or seqlen_q > 1) a grouped
// variant takes up to eight of them per workgroup, so each key row is loaded once
// for all of them.
//
// Combine kernel: out = sum_s exp(lse_s - L) out_s with L = ln sum_s exp(lse_s).
#include "fa_common.h"

namespace fa {

constexpr int DEC_THREADS = 256;
#ifndef FA_DEC_UNROLL
#define FA_DEC_UNROLL 8
#endif
#ifndef FA_DEC_CPOL
#define FA_DEC_CPOL 2
#endif
constexpr int DEC_UNROLL = FA_DEC_UNROLL;  // key rows per lane per step
constexpr int DEC_CPOL = FA_DEC_CPOL;      // KV loads are non-temporal (read once, streamed)


// KVC: the keys come from a KV cache (fa_fwd_kvcache): sequence b has
// cache_seqlens[b] + seqlen_new keys, block n of it lives in block block_table[b, n]
// (or block b of a contiguous cache), and K/V may have fewer heads than Q.
template <int HD, bool ALIBI, bool KVC, typename E>
__global__ __launch_bounds__(DEC_THREADS) void decode_split_kernel(FwdParams p) {
  constexpr int LPR = HD / 8;    // lanes per key row
  constexpr int RPW = 64 / LPR;  // key rows per wave per load
  constexpr int STEP = DEC_UNROLL * RPW;
  __shared__ float sm_m[4], sm_l[4];
  __shared__ float sm_acc[4][HD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane / LPR;   // row group inside the wave
  const int cidx = lane % LPR;  // 8-column chunk of the head dimension

  int w = xcd_remap(blockIdx.x, gridDim.x);
  const int Sq = p.seqlen_q;
  const int i = w % Sq;
  w /= Sq;
  const int split = w % p.num_splits;
  w /= p.num_splits;
  const int h = w % p.nheads;
  const int b = w / p.nheads;
  const int Sk = KVC ? p.cache_seqlens[b] + p.seqlen_new : p.seqlen_k;

  const long row_stride = (long)p.nheads * HD;       // q
  const long kv_stride = (long)p.nheads_k * HD;      // k, v
  const int row_bytes = (int)kv_stride * 2;
  const int hk = h / (p.nheads / p.nheads_k);

  // visible keys of row i inside this split: [lo, hi)
  const int pos = i + Sk - Sq;
  int lo = min(Sk, split * p.split_len);
  int hi = min(Sk, lo + p.split_len);
  if (p.window_left >= 0) lo = max(lo, pos - p.window_left);
  if (p.window_right >= 0) hi = min(hi, pos + p.window_right + 1);
  const long kvb = KVC ? (long)hk * HD : (long)b * Sk * kv_stride + (long)hk * HD;  // key 0 / head offset
  // KV-cache steps start on multiples of STEP so that none crosses a block; keys
  // below lo are then masked
  const int first = KVC ? (lo & ~(STEP - 1)) : lo;

  // q chunk, pre-multiplied by softmax_scale * log2(e) (sign included)
  const float c = (p.q_sign ? -p.scale_log2 : p.scale_log2);
  float qv[8];
  {
    const u32x4 raw = *(const u32x4*)(p.q + ((long)b * Sq + i) * row_stride + (long)h * HD + cidx * 8) & p.q_and;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = widen_lo<E>(raw[e]) * c;
      qv[2 * e + 1] = widen_hi<E>(raw[e]) * c;
    }
  }
  float slope = 0.f;
  if constexpr (ALIBI) slope = p.alibi[(long)b * p.alibi_bstride + h] * kLog2e;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  for (int base = first + wave * STEP; base < hi; base += 4 * STEP) {
    // buffer resources over keys [base, min(hi, base + STEP)): later keys read as zeros
    const int nrec = min(hi - base, STEP) * row_bytes;
    long row0 = base;  // physical row of key `base`
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
    u32x4 kr[DEC_UNROLL], vr[DEC_UNROLL];
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u) {
      const int off = (u * RPW + g) * row_bytes + cidx * 16;
      kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, DEC_CPOL));
      vr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, DEC_CPOL));
    }
    float s[DEC_UNROLL];
    float bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fmaf(qv[2 * e], widen_lo<E>(kr[u][e]), part);
        part = fmaf(qv[2 * e + 1], widen_hi<E>(kr[u][e]), part);
      }
#pragma unroll
      for (int o = LPR / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
      const int key = base + u * RPW + g;
      if constexpr (ALIBI) part -= slope * fabsf((float)(pos - key));
      s[u] = (key < hi && (!KVC || key >= lo)) ? part : -INFINITY;
      bmax = fmaxf(bmax, s[u]);
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o));

    const float m_new = fmaxf(m_run, bmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u) {
      const float pu = fast_exp2(s[u] - m_use);
      l_run += pu;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(pu, widen_lo<E>(vr[u][e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(pu, widen_hi<E>(vr[u][e]), acc[2 * e + 1]);
      }
    }
    m_run = m_new;
  }

  // merge the row groups of this wave (same m_run across the wave)
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
    l_run += __shfl_xor(l_run, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o);
  }
  if (lane == 0) {
    sm_m[wave] = m_run;
    sm_l[wave] = l_run;
  }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[wave][cidx * 8 + e] = acc[e];
  }
  __syncthreads();

  // merge the four waves
  float M = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
  const float M_use = (M == -INFINITY) ? 0.f : M;
  float wgt[4], L = 0.f;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    wgt[x] = fast_exp2(sm_m[x] - M_use);
    L += sm_l[x] * wgt[x];
  }
  const long rowid = (((long)split * p.batch + b) * p.nheads + h) * Sq + i;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* out = (float*)p.out + rowid * HD;
  for (int d = tid; d < HD; d += DEC_THREADS) {
    float o = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) o = fmaf(sm_acc[x][d], wgt[x], o);
    out[d] = o * inv;
  }
  if (tid == 0) p.lse[rowid] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
}

// Grouped decode partial kernel: one workgroup per (batch, K/V head, split, chunk of
// NQ queries).  The queries of a K/V head are its nheads / nheads_k query heads times
// the seqlen_q rows (query n: head hk * G + n / Sq, row n % Sq); one workgroup takes NQ
// of them, so each key row it loads serves NQ dot products instead of one.  Each
// query keeps its own visible range, ALiBi slope and online-softmax state.
template <int HD, bool ALIBI, bool KVC, int NQ, typename E>
__global__ __launch_bounds__(DEC_THREADS) void decode_group_kernel(FwdParams p) {
  constexpr int LPR = HD / 8;
  constexpr int RPW = 64 / LPR;
  constexpr int UNROLL = NQ <= 2 ? DEC_UNROLL : DEC_UNROLL / 2;  // registers: NQ copies of the state
  constexpr int STEP = UNROLL * RPW;
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
  float qv[NQ][8], slope[NQ];
  int q_lo[NQ], q_hi[NQ], q_pos[NQ];
  int lo = s_hi, hi = s_lo;  // union of the queries' visible ranges in this split
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
    const u32x4 raw = valid ? *(const u32x4*)(p.q + ((long)b * Sq + i) * row_stride + (long)h * HD + cidx * 8) & p.q_and
                            : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[j][2 * e] = widen_lo<E>(raw[e]) * c;
      qv[j][2 * e + 1] = widen_hi<E>(raw[e]) * c;
    }
    slope[j] = 0.f;
    if constexpr (ALIBI) slope[j] = p.alibi[(long)b * p.alibi_bstride + h] * kLog2e;
  }
  if (hi <= lo) lo = hi = 0;  // no query sees a key of this split
  const long kvb = KVC ? (long)hk * HD : (long)b * Sk * kv_stride + (long)hk * HD;
  const int first = KVC ? (lo & ~(STEP - 1)) : lo;

  float m_run[NQ], l_run[NQ], acc[NQ][8];
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
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float sj[UNROLL];
      float bmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part = fmaf(qv[j][2 * e], widen_lo<E>(kr[u][e]), part);
          part = fmaf(qv[j][2 * e + 1], widen_hi<E>(kr[u][e]), part);
        }
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
        const int key = base + u * RPW + g;
        if constexpr (ALIBI) part -= slope[j] * fabsf((float)(q_pos[j] - key));
        sj[u] = (key >= q_lo[j] && key < q_hi[j]) ? part : -INFINITY;
        bmax = fmaxf(bmax, sj[u]);
      }
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o));
      const float m_new = fmaxf(m_run[j], bmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[j] - m_use);
      l_run[j] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= alpha;
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
      m_run[j] = m_new;
    }
  }

  // merge the row groups of each wave, then the four waves, per query
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
      l_run[j] += __shfl_xor(l_run[j], o);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] += __shfl_xor(acc[j][e], o);
    }
    if (lane == 0) {
      sm_m[wave][j] = m_run[j];
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

template <int HD, typename E>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int PER_LANE = HD / 64;
  const int lane = threadIdx.x & 63;
  const long rows = (long)p.batch * p.nheads * p.seqlen_q;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*H + h)*Sq + i
  if (row >= rows) return;
  const int i = (int)(row % p.seqlen_q);
  const long bh = row / p.seqlen_q;
  const int h = (int)(bh % p.nheads);
  const int b = (int)(bh / p.nheads);

  const float* lp = p.lse_partial + row;
  const float* op = p.out_partial + row * HD;
  const long lstride = rows, ostride = rows * HD;

  float M = -INFINITY;
  for (int s = 0; s < p.num_splits; ++s) M = fmaxf(M, lp[s * lstride]);

  float o[PER_LANE];
#pragma unroll
  for (int e = 0; e < PER_LANE; ++e) o[e] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < p.num_splits; ++s) {
      const float ls = lp[s * lstride];
      const float wgt = fast_exp2((ls - M) * kLog2e);  // 0 for an empty split
      L += wgt;
      if (wgt != 0.f) {
#pragma unroll
        for (int e = 0; e < PER_LANE; ++e) o[e] = fmaf(wgt, op[s * ostride + lane + 64 * e], o[e]);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* out = p.out + (((long)b * p.seqlen_q + i) * p.nheads + h) * HD;
#pragma unroll
  for (int e = 0; e < PER_LANE; ++e) {
    const uint32_t pk = pack2<E>(o[e] * inv, 0.f);
    out[lane + 64 * e] = (uint16_t)(pk & 0xffffu);
  }
  if (lane == 0) p.lse[row] = L > 0.f ? M + logf(L) : -INFINITY;
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

// Queries one decode workgroup serves when a K/V head has nq_total of them.
int decode_queries_per_block(int nq_total) { return nq_total <= 1 ? 1 : nq_total <= 2 ? 2 : nq_total <= 4 ? 4 : 8; }

template <int HD, bool ALIBI, bool KVC, typename E>
static void launch_group_nq(const FwdParams& p, hipStream_t stream) {
  switch (decode_queries_per_block(p.nheads / p.nheads_k * p.seqlen_q)) {
    case 2: launch_group<HD, ALIBI, KVC, 2, E>(p, stream); break;
    case 4: launch_group<HD, ALIBI, KVC, 4, E>(p, stream); break;
    default: launch_group<HD, ALIBI, KVC, 8, E>(p, stream); break;
  }
}

template <int HD, bool KVC, typename E>
static hipError_t launch_decode_kvc(const FwdParams& p, hipStream_t stream) {
  // several queries per K/V head (grouped heads or seqlen_q > 1): the grouped kernel
  // loads each key row once for all of them
  if (p.nheads / p.nheads_k * p.seqlen_q > 1) {
    if (p.alibi) launch_group_nq<HD, true, KVC, E>(p, stream);
    else launch_group_nq<HD, false, KVC, E>(p, stream);
    return hipGetLastError();
  }
  const long nblocks = (long)p.batch * p.nheads * p.num_splits * p.seqlen_q;
  if (p.alibi)
    hipLaunchKernelGGL((decode_split_kernel<HD, true, KVC, E>), dim3((unsigned)nblocks), dim3(DEC_THREADS), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<HD, false, KVC, E>), dim3((unsigned)nblocks), dim3(DEC_THREADS), 0,
                       stream, p);
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

// Key rows one decode step covers per wave (blocks of a paged cache must hold a whole
// number of them): DEC_UNROLL * 64 / (headdim / 8).
int decode_step_keys(int headdim) { return DEC_UNROLL * 64 / (headdim / 8); }

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
  const dim3 grid((unsigned)((rows + 3) / 4));
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
