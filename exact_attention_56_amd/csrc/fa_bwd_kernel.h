// fa_bwd_kernel.h - matrix-core (MFMA) attention backward for gfx950 (kernel templates;
// fa_bwd.hip instantiates them).
//
// What it computes, per (batch, head), for the visible (query i, key j) pairs:
//   P_ij = exp(scale * q_i.k_j + bias_ij - L_i)       (L = the forward's logsumexp)
//   dV_j = sum_i P_ij dO_i,          dP_ij = dO_i . v_j,
//   D_i  = dO_i . O_i,               dS_ij = P_ij (dP_ij - D_i),
//   dQ_i = scale * sum_j dS_ij k_j,  dK_j  = scale * sum_i dS_ij q_i,
// following the page "FlashAttention：快速且内存高效的准确注意力机制"
// (cloud.tencent.com.cn/developer/article/2433927), sections "算法 / 反向传播" (P is
// recomputed from the row-wise logsumexp alone, same tiling as the forward) and
// "并行性 / 反向传播" (one block per column block of K and V).
//
// Design for CDNA4:
//  * two kernels, run in this order: dq_kernel (one workgroup per 128 queries: Q and
//    dO stay in registers while 64-key tiles of K and V stream through LDS; it also
//    forms D = rowsum(dO o O) of its rows in fp32 and writes it out) and dkdv_kernel
//    (one workgroup per 128 keys of a (batch, head): K and V of its keys stay in
//    registers while query tiles of Q, dO, L, D stream through LDS).  dQ gets its own
//    pass instead of atomic adds from the key-block workgroups: every output element
//    is written once, so the results are deterministic, and no fp32 accumulation
//    buffer is needed;
//  * all products are v_mfma_f32_32x32x16_bf16 with transposed outputs where that
//    keeps row statistics lane-local: the dq kernel holds S^T, dP^T (lane = query),
//    the dkdv kernel S, dP (lane = key);
//  * an accumulator whose rows are the contraction index of the next product is
//    used directly as that product's B operand (rounded to bf16): the A operand of
//    the first product reads LDS rows with bits 2 and 3 of the row index swapped,
//    which puts 8 consecutive rows in each lane's registers;
//  * the streamed tiles stay in their natural row order in LDS: the same tile
//    serves the row reads (ds_read_b128, permuted rows) and the transposed reads
//    (ds_read_b64_tr_b16) of the second product.
#pragma once
#include "fa_fwd_kernel.h"

namespace fa {

constexpr int BWD_NW = 4;        // waves per workgroup
constexpr int DQ_TILE = 64;      // keys per streamed tile (dq kernel)
// Queries per streamed tile (dkdv kernel): 32.  Headdim 64 keeps two waves per SIMD that
// way; headdim 256 runs one wave per SIMD (K and V of 32 keys fill 128 registers, dK and dV
// 256).  Headdim 128 without V in LDS (below) takes 64: two independent 32-query blocks per
// wave at one wave per SIMD.
#ifndef FA_DKV_TILE128
#define FA_DKV_TILE128 64
#endif
// Headdim 128 with V in LDS (VLDS): each wave keeps only K of its 32 keys in registers and
// reads V from one LDS copy of the workgroup's 128 keys; with 32-query tiles the kernel then
// fits two waves per SIMD, where one wave per SIMD left it bound by the LDS reads one wave
// can receive.
#ifndef FA_DKV_VLDS
#define FA_DKV_VLDS 1
#endif
template <int HD>
constexpr bool dkv_vlds() { return HD == 128 && FA_DKV_VLDS; }
template <int HD>
constexpr int dkv_tile() { return HD == 128 ? (dkv_vlds<HD>() ? 32 : FA_DKV_TILE128) : 32; }

// Two bf16 [rows][row_stride] tensors streamed tile by tile (ROWS rows) into LDS in
// natural row order, rows SA (SB) 16-byte slots apart; direct-to-LDS buffer loads,
// rows past `hi` and pad slots land as zeros.  Load u of a tile (wave u % NW issues
// it) fills LDS bytes [1024u, 1024u + 1024).
template <int HD, int ROWS, int SA, int SB>
struct PairStream {
  static constexpr int CPR = HD / 8;
  static constexpr int LA = (ROWS * SA + 63) / 64, LB = (ROWS * SB + 63) / 64;
  static constexpr int PWA = (LA + BWD_NW - 1) / BWD_NW, PWB = (LB + BWD_NW - 1) / BWD_NW;
  static constexpr int ABYTES = 1024 * LA, BBYTES = 1024 * LB;  // loads wholly past a tile are not issued
  static_assert(SA >= CPR && SB >= CPR, "a row holds its chunks");
  const uint16_t* abase;
  const uint16_t* bbase;
  int lo, hi, row_stride, row_bytes, lw;
  uint32_t aoff[PWA], boff[PWB];

  __device__ __forceinline__ void init(int wave, int lane) {
    lw = wave;
#pragma unroll
    for (int i = 0; i < PWA; ++i) {
      const int slot = 64 * (lw + BWD_NW * i) + lane;
      const int row = slot / SA, ch = slot % SA;
      aoff[i] = (row < ROWS && ch < CPR) ? (uint32_t)(row * row_bytes + ch * 16) : OOB_OFFSET;
    }
#pragma unroll
    for (int i = 0; i < PWB; ++i) {
      const int slot = 64 * (lw + BWD_NW * i) + lane;
      const int row = slot / SB, ch = slot % SB;
      boff[i] = (row < ROWS && ch < CPR) ? (uint32_t)(row * row_bytes + ch * 16) : OOB_OFFSET;
    }
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t* base, int t) const {
    const int j0 = lo + t * ROWS;
    const int rows = hi - j0;
    const int n = rows > 0 ? min(rows, ROWS) * row_bytes : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (long)j0 * row_stride), (short)0, n, 0x00020000);
  }
  __device__ __forceinline__ void load(lds_u8* dsta, lds_u8* dstb, int t) const {
    const auto ra = rsrc(abase, t);
#pragma unroll
    for (int i = 0; i < PWA; ++i)
      if (lw + BWD_NW * i < LA)  // loads wholly past the tile are skipped (wave-uniform)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dsta + 1024 * (lw + BWD_NW * i), 16, (int)aoff[i], 0, 0, 0);
    const auto rb = rsrc(bbase, t);
#pragma unroll
    for (int i = 0; i < PWB; ++i)
      if (lw + BWD_NW * i < LB)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dstb + 1024 * (lw + BWD_NW * i), 16, (int)boff[i], 0, 0, 0);
  }
};

// A operand (32 rows x 16 columns) read from a row-major LDS tile: lane l takes row
// k_lds_row(l % 32) + 32 blk, 16 bytes at column 16 kk + 8 (l / 32).
template <int PITCH, typename E>
__device__ __forceinline__ x8<E> row_operand(const lds_u8* tile, int lrow, int half, int blk, int kk) {
  return *(const __attribute__((address_space(3))) x8<E>*)(tile + (k_lds_row(lrow) + 32 * blk) * PITCH + 32 * kk +
                                                            16 * half);
}

// A operand of a transposed product: X^T[d][rows 16 ci + 8 (l / 32) + 0..7] for
// d = 32 db + l % 32, from a row-major LDS tile (two transpose reads; see
// vt_lane_offset for the lane pattern, here with any row pitch).
template <int PITCH, typename E>
__device__ __forceinline__ x8<E> tr_operand(const lds_u8* tile, int lane, int db, int ci) {
  const int g = lane >> 4, r = lane & 15;
  const lds_u8* p = tile + (8 * (g >> 1) + (r >> 2)) * PITCH + (16 * (g & 1) + 4 * (r & 3)) * 2;
  const s16x4 lo = lds_read_tr(p + 16 * ci * PITCH + 64 * db);
  const s16x4 hi = lds_read_tr(p + (16 * ci + 4) * PITCH + 64 * db);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(x8<E>, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 16 bytes of row `row` of a [rows][row_stride] 16-bit tensor as a B operand (8
// consecutive columns starting at 16 kk + 8 half), zero past the last row.
template <typename E>
__device__ __forceinline__ x8<E> row_fragment(const uint16_t* base, long row_stride, int row, int nrows, int kk,
                                               int half, uint32_t and_mask, uint32_t xor_mask) {
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (row < nrows) raw = *(const u32x4*)(base + (long)row * row_stride + 16 * kk + 8 * half);
  raw = (raw & and_mask) ^ xor_mask;
  return __builtin_bit_cast(x8<E>, raw);
}

// Pack register pairs (2e, 2e+1) of 8 consecutive accumulator rows r0..r0+7 into the
// B operand (element type E) of the next product.
template <typename E>
__device__ __forceinline__ x8<E> pack_rows(const f32x16& x, int r0) {
  return __builtin_bit_cast(x8<E>, u32x4{pack2<E>(x[r0], x[r0 + 1]), pack2<E>(x[r0 + 2], x[r0 + 3]),
                                         pack2<E>(x[r0 + 4], x[r0 + 5]), pack2<E>(x[r0 + 6], x[r0 + 7])});
}

// Store a transposed accumulator X^T [HD rows (d) x 32 columns] of this wave as E
// row `row` (the lane's column) of a [rows][row_stride] tensor, times `mul`.
template <int HD, typename E>
__device__ __forceinline__ void store_rows(uint16_t* base, long row_stride, int row, const f32x16 (&x)[HD / 32],
                                                float mul, int half) {
  uint16_t* o = base + (long)row * row_stride;
#pragma unroll
  for (int db = 0; db < HD / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // accumulator rows 4g..4g+3 of block db hold columns 32db + 8g + 4*half + 0..3
      const int d0 = 32 * db + 8 * g + 4 * half;
      u32x2 w = {pack2<E>(x[db][4 * g] * mul, x[db][4 * g + 1] * mul),
                 pack2<E>(x[db][4 * g + 2] * mul, x[db][4 * g + 3] * mul)};
      *(u32x2*)(o + d0) = w;
    }
}

// Rows of sequence b: the first q and k row and the lengths; padded batches use the
// common lengths.  The first lse/delta element of (b, h) is lse_row(p, b, h, q_start, Sq).
struct SeqRows {
  long q_start, k_start;
  int Sq, Sk;
};
__device__ __forceinline__ SeqRows seq_rows(const BwdParams& p, int b) {
  SeqRows r;
  if (p.cu_q != nullptr) {
    r.q_start = p.cu_q[b];
    r.Sq = p.cu_q[b + 1] - (int)r.q_start;
    r.k_start = p.cu_k[b];
    r.Sk = p.cu_k[b + 1] - (int)r.k_start;
  } else {
    r.Sq = p.seqlen_q;
    r.Sk = p.seqlen_k;
    r.q_start = (long)b * r.Sq;
    r.k_start = (long)b * r.Sk;
  }
  return r;
}
__device__ __forceinline__ long lse_row(const BwdParams& p, int b, int h, const SeqRows& r) {
  return p.cu_q != nullptr ? (long)h * p.lse_head_stride + r.q_start : ((long)b * p.nheads + h) * r.Sq;
}

// Bias in log2 units of query i and key j (ALiBi), or 0.
__device__ __forceinline__ float alibi_log2(float slope_log2, int pos_i, int key) {
  return -slope_log2 * fabsf((float)(pos_i - key));
}

// ---------------------------------------------------------------------------------
// dq_kernel: one workgroup per (batch, head, 128 queries); wave w owns queries
// i0 + 32 w + 0..31.  Per 64-key tile t:
//   S^T = K Q^T, dP^T = V dO^T   (lane = query; K, V rows from LDS, Q, dO in registers)
//   P^T = exp2(S^T c + bias - L'), dS^T = P^T (dP^T - D)
//   dQ^T += K^T dS^T              (K^T by transpose reads, dS^T as the B operand)
template <int HD, bool ALIBI, typename E>
__global__ __launch_bounds__(256) void dq_kernel(BwdParams p, int items) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass needs only the signature
  constexpr int KS = HD / 8 + 2;  // K rows: transpose reads dominate (V-style pitch)
  constexpr int VS = HD / 8 + 1;  // V rows: row reads only (K-style pitch)
  using Stream = PairStream<HD, DQ_TILE, KS, VS>;
  constexpr int KP = KS * 16, VP = VS * 16;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (Stream::ABYTES + Stream::BBYTES)];
  lds_u8* const lds = (lds_u8*)smem;
  // buffer i: K at lds + i * ABYTES, V at lds + 2 * ABYTES + i * BBYTES

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, half = lane >> 5;

  // Padded batch with a causal mask or right window: later query tiles see more keys.
  // Each XCD's range then runs in groups of up to four (batch, head) pairs, query tile
  // slowest and heaviest first inside a group (as in the forward).  Otherwise tiles run
  // fastest within the XCD-contiguous ranges of xcd_remap, head slowest: on a packed
  // batch each XCD then takes a slice of the heads over every sequence (equal work
  // whatever the lengths; grouping sequences instead left the XCDs unequal and ran at
  // 58% of this order's speed), heaviest tile of each sequence first under a mask.
  int qt, b, h;
  if (p.window_right >= 0 && p.cu_q == nullptr) {
    const int bh = heavy_first_item(xcd_remap(blockIdx.x, items), p.num_q_tiles, p.batch * p.nheads, qt);
    qt = p.num_q_tiles - 1 - qt;
    b = bh % p.batch;
    h = bh / p.batch;
  } else {
    int w = xcd_remap(blockIdx.x, items);
    qt = w % p.num_q_tiles;
    w /= p.num_q_tiles;
    b = w % p.batch;
    h = w / p.batch;
    if (p.window_right >= 0) qt = p.num_q_tiles - 1 - qt;  // packed: heaviest tile of a sequence first
  }

  const SeqRows sr = seq_rows(p, b);
  const int Sq = sr.Sq, Sk = sr.Sk, off = Sk - Sq;
  if (qt * BWD_ROWS >= Sq) return;  // the whole workgroup: a packed sequence shorter than the tile
  const int wl = p.window_left, wr = p.window_right;
  const long rs = (long)p.nheads * HD, rsk = (long)p.nheads_k * HD;
  const int hk = h / (p.nheads / p.nheads_k);
  const long qoff = sr.q_start * rs + (long)h * HD, koff = sr.k_start * rsk + (long)hk * HD;

  const int i0 = qt * BWD_ROWS;
  const int i_last = min(i0 + BWD_ROWS, Sq) - 1;
  const int my_q = i0 + 32 * wave + lrow;
  const int my_pos = my_q + off;

  // key tiles any row of this block sees
  int lo = 0, hi = Sk - 1;
  if (wl >= 0) lo = max(lo, i0 + off - wl);
  if (wr >= 0) hi = min(hi, i_last + off + wr);
  const int t_begin = hi >= lo ? lo / DQ_TILE : 0;
  const int t_end = hi >= lo ? hi / DQ_TILE + 1 : 0;

  // the first K/V tile is on its way to LDS while this wave loads its rows and forms D
  Stream st;
  st.abase = p.k + koff;
  st.bbase = p.v + koff;
  st.lo = 0;
  st.hi = Sk;
  st.row_stride = (int)rsk;
  st.row_bytes = (int)rsk * 2;
  st.init(wave, lane);
  if (t_begin < t_end) st.load(lds, lds + 2 * Stream::ABYTES, t_begin);

  x8<E> qf[HD / 16], gf[HD / 16];
#pragma unroll
  for (int kk = 0; kk < HD / 16; ++kk) {
    qf[kk] = row_fragment<E>(p.q + qoff, rs, my_q, Sq, kk, half, p.q_and, p.q_sign);
    gf[kk] = row_fragment<E>(p.dout + qoff, rs, my_q, Sq, kk, half, 0xffffffffu, 0u);
  }
  // D = rowsum(dO o O) of this lane's row in fp32: the lane holds half of the row's dO
  // (gf) and reads the same half of O; the other half-wave holds the rest.  Written to
  // delta for the dK/dV pass, which runs after this one.
  float dpart = 0.f;
  if (my_q < Sq) {
    const uint16_t* orow = p.out + qoff + (long)my_q * rs;
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) {
      const u32x4 o = *(const u32x4*)(orow + 16 * kk + 8 * half);
      const u32x4 g = __builtin_bit_cast(u32x4, gf[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dpart = fmaf(widen_lo<E>(o[e]), widen_lo<E>(g[e]), dpart);
        dpart = fmaf(widen_hi<E>(o[e]), widen_hi<E>(g[e]), dpart);
      }
    }
  }
  const float drow = sum_with_other_half(dpart);
  // L in log2 units (an empty row gets +inf, so that every P of it is 0)
  float lrow2 = INFINITY;
  if (my_q < Sq) {
    const long li = lse_row(p, b, h, sr) + my_q;
    const float l = p.lse[li];
    lrow2 = l == -INFINITY ? INFINITY : l * kLog2e;
    if (half == 0) p.delta[li] = drow;
  }
  const float c = p.scale_log2;
  float slope2 = 0.f;
  if constexpr (ALIBI) slope2 = p.alibi[(long)b * p.alibi_bstride + h] * kLog2e;

  f32x16 dq[HD / 32];
#pragma unroll
  for (int db = 0; db < HD / 32; ++db) dq[db] = f32x16{};

  // One key tile: S^T, dP^T, then P^T and dS^T, then dQ^T.  MODE 0: every pair visible;
  // 1: with the mask (a mask boundary or the end crosses the tile); 2: no key of the tile
  // is visible to this wave: only its share of the loads and the barrier.
  auto step = [&](int t, auto mode) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool MASKED = MODE == 1;
    const int cur = (t - t_begin) & 1;
    wait_tile_loads<0>();
    __syncthreads();  // tile t is in LDS; everyone is done with the other buffer
    if (t + 1 < t_end)
      st.load(lds + (cur ^ 1) * Stream::ABYTES, lds + 2 * Stream::ABYTES + (cur ^ 1) * Stream::BBYTES, t + 1);
    if constexpr (MODE == 2) return;
    const lds_u8* kt = lds + cur * Stream::ABYTES;
    const lds_u8* vt = lds + 2 * Stream::ABYTES + cur * Stream::BBYTES;

    f32x16 s[2], dp[2];
    s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma32(row_operand<KP, E>(kt, lrow, half, kb, kk), qf[kk], s[kb]);
        dp[kb] = mfma32(row_operand<VP, E>(vt, lrow, half, kb, kk), gf[kk], dp[kb]);
      }

    // P^T and dS^T.  Register r of block kb holds key j0 + 32 kb + 16 (r / 8) + 8 half + r % 8.
    const int j0 = t * DQ_TILE;
    int vlo = 0, vspan = -1;  // visible keys of this row: [vlo, vlo + vspan]
    if constexpr (MASKED) {
      const int klo = wl < 0 ? 0 : max(0, my_pos - wl);
      const int khi = wr < 0 ? Sk - 1 : min(Sk - 1, my_pos + wr);
      vlo = klo;
      vspan = khi - klo;
    }
    x8<E> dsf[4];
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) {
      const int kb = ci >> 1, r0 = 8 * (ci & 1);
      f32x16 tmp;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = j0 + 32 * kb + 16 * (r0 / 8) + 8 * half + e;
        float x = fmaf(s[kb][r0 + e], c, -lrow2);
        if constexpr (ALIBI) x += alibi_log2(slope2, my_pos, key);
        float pv = fast_exp2(x);
        if constexpr (MASKED) {
          const bool vis = vspan >= 0 && (uint32_t)(key - vlo) <= (uint32_t)vspan && my_q < Sq;
          pv = vis ? pv : 0.f;
        }
        tmp[e] = pv * (dp[kb][r0 + e] - drow);
      }
      dsf[ci] = pack_rows<E>(tmp, 0);
    }

    // dQ^T += K^T dS^T
#pragma unroll
    for (int ci = 0; ci < 4; ++ci)
#pragma unroll
      for (int db = 0; db < HD / 32; ++db)
        dq[db] = mfma32(tr_operand<KP, E>(kt, lane, db, ci), dsf[ci], dq[db]);
  };
  // The tiles every (query of this wave, key) pair of which is visible, with no key past
  // the end, form one range [tf_begin, tf_end): run there without the mask, in a loop of
  // its own, as in dkdv_kernel; the tiles with any key visible to the wave form a range
  // [tv_begin, tv_end) around it, and outside that the wave only loads and meets the
  // barrier (under a causal mask the block's first rows see one 64-key tile fewer than
  // its last).  Every wave passes the same number of steps.
  const int wi0 = min(i0 + 32 * wave, Sq - 1), wil = min(i0 + 32 * wave + 31, Sq - 1);
  const int kvlo = wl < 0 ? 0 : max(0, wi0 + off - wl), kvhi = wr < 0 ? Sk - 1 : min(Sk - 1, wil + off + wr);
  const int tv_begin = kvhi < kvlo ? t_end : min(max(t_begin, kvlo / DQ_TILE), t_end);
  const int tv_end = kvhi < kvlo ? t_end : max(tv_begin, min(t_end, kvhi / DQ_TILE + 1));
  int tf_lo = 0, tf_hi = Sk / DQ_TILE;  // full tiles: tf_lo <= t < tf_hi
  if (wl >= 0) {
    const int x = wil + off - wl;  // needs t * DQ_TILE >= x
    tf_lo = x <= 0 ? 0 : (x + DQ_TILE - 1) / DQ_TILE;
  }
  if (wr >= 0) {
    const int y = wi0 + off + wr - DQ_TILE + 1;  // needs t * DQ_TILE <= y
    tf_hi = min(tf_hi, y < 0 ? 0 : y / DQ_TILE + 1);
  }
  const int tf_begin = min(max(tv_begin, tf_lo), tv_end);
  const int tf_end = max(tf_begin, min(tv_end, tf_hi));
  int t = t_begin;
  for (; t < tv_begin; ++t) step(t, std::integral_constant<int, 2>{});
  for (; t < tf_begin; ++t) step(t, std::integral_constant<int, 1>{});
  for (; t < tf_end; ++t) step(t, std::integral_constant<int, 0>{});
  for (; t < tv_end; ++t) step(t, std::integral_constant<int, 1>{});
  for (; t < t_end; ++t) step(t, std::integral_constant<int, 2>{});
  if (my_q < Sq) store_rows<HD, E>(p.dq + qoff, rs, my_q, dq, p.scale, half);
#endif
}

// ---------------------------------------------------------------------------------
// dkdv_kernel: one workgroup per (batch, K/V head, 128 keys); wave w owns keys
// j0 + 32 w + 0..31.  For each query head that reads the K/V head, per query tile t:
//   S = Q K^T, dP = dO V^T        (lane = key; Q, dO rows from LDS, K, V in registers)
//   P = exp2(S c + bias - L'), dS = P (dP - D)
//   dV^T += dO^T P, dK^T += Q^T dS   (dO^T, Q^T by transpose reads; P, dS as B operands)
template <int HD, bool ALIBI, typename E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(dkv_vlds<HD>() ? 2 : 1))) void dkdv_kernel(
    BwdParams p, int items) {
  constexpr int DKV_TILE = dkv_tile<HD>(), DKV_QB = DKV_TILE / 32;
  constexpr bool VLDS = dkv_vlds<HD>();
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass needs only the signature
  constexpr int QS = HD / 8 + 2;  // Q and dO rows: both read both ways
  using Stream = PairStream<HD, DKV_TILE, QS, QS>;
  constexpr int QP = QS * 16;
  constexpr int LDBYTES = 256;    // L' and D of one tile (fp32, 64 lanes x 4 bytes each)
  constexpr int VP = (HD / 8 + 1) * 16;  // VLDS: bytes per V row in LDS (16-byte reads, no conflicts)
  constexpr int VBYTES = VLDS ? BWD_ROWS * VP : 0;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (Stream::ABYTES + Stream::BBYTES + 2 * LDBYTES) + VBYTES];
  lds_u8* const lds = (lds_u8*)smem;
  // buffer i at lds + i * BUF: Q tile, dO tile, then L and D; VLDS: V of the keys after both
  constexpr int BUF = Stream::ABYTES + Stream::BBYTES + 2 * LDBYTES;
  constexpr int GOFF = Stream::ABYTES, LOFF = Stream::ABYTES + Stream::BBYTES, VOFF = 2 * BUF;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, half = lane >> 5;

  // Work items are (batch, K/V head, key tile).  Padded batch with a causal mask or
  // right window: earlier key tiles are seen by more queries; they run first within
  // each group of (batch, K/V head) pairs, as in dq_kernel.  Otherwise (and for packed
  // batches) key tile fastest, K/V head slowest, as in dq_kernel.
  int kt_idx, b, hk;
  if (p.window_right >= 0 && p.cu_q == nullptr) {
    const int bh = heavy_first_item(xcd_remap(blockIdx.x, items), p.num_k_tiles, p.batch * p.nheads_k, kt_idx);
    b = bh % p.batch;
    hk = bh / p.batch;
  } else {
    int w = xcd_remap(blockIdx.x, items);
    kt_idx = w % p.num_k_tiles;
    w /= p.num_k_tiles;
    b = w % p.batch;
    hk = w / p.batch;
  }

  const SeqRows sr = seq_rows(p, b);
  const int Sq = sr.Sq, Sk = sr.Sk, off = Sk - Sq;
  if (kt_idx * BWD_ROWS >= Sk) return;  // the whole workgroup: a packed sequence shorter than the tile
  const int wl = p.window_left, wr = p.window_right;
  const long rs = (long)p.nheads * HD, rsk = (long)p.nheads_k * HD;
  const long koff = sr.k_start * rsk + (long)hk * HD;
  const int group = p.nheads / p.nheads_k;

  const int j0 = kt_idx * BWD_ROWS;
  const int j_last = min(j0 + BWD_ROWS, Sk) - 1;
  const int my_k = j0 + 32 * wave + lrow;

  // query tiles that see any key of this block: c_i = i + off in [j0 - wr, j_last + wl]
  int lo = 0, hi = Sq - 1;
  if (wr >= 0) lo = max(lo, j0 - wr - off);
  if (wl >= 0) hi = min(hi, j_last + wl - off);
  const int t_begin = hi >= lo ? lo / DKV_TILE : 0;
  const int t_end = hi >= lo ? hi / DKV_TILE + 1 : 0;

  x8<E> kf[HD / 16], vf[VLDS ? 1 : HD / 16];
  // VLDS: this lane's 16-byte slots of its key's V row in LDS (B operand of dP = dO V^T)
  const lds_u8* const vrow = lds + VOFF + (32 * wave + lrow) * VP + 16 * half;
#pragma unroll
  for (int kk = 0; kk < HD / 16; ++kk) {
    kf[kk] = row_fragment<E>(p.k + koff, rsk, my_k, Sk, kk, half, p.q_and, p.q_sign);
    const x8<E> v = row_fragment<E>(p.v + koff, rsk, my_k, Sk, kk, half, 0xffffffffu, 0u);
    if constexpr (VLDS)
      *(__attribute__((address_space(3))) x8<E>*)(lds + VOFF + (32 * wave + lrow) * VP + 16 * half + 32 * kk) = v;
    else
      vf[kk] = v;
  }
  // (the first tile's barrier orders these stores before any read)
  const float c = p.scale_log2;
  // visible queries of this key: c_i in [my_k - wr, my_k + wl]
  const int qlo = wr < 0 ? 0 : max(0, my_k - wr - off);
  const int qhi = wl < 0 ? Sq - 1 : min(Sq - 1, my_k + wl - off);

  f32x16 dk[HD / 32], dv[HD / 32];
#pragma unroll
  for (int db = 0; db < HD / 32; ++db) dk[db] = dv[db] = f32x16{};

  // The query heads that read this K/V head, one after another: dK and dV sum their
  // contributions in the same accumulators.
  for (int h = hk * group; h < (hk + 1) * group; ++h) {
    const long qoff = sr.q_start * rs + (long)h * HD;
    const long loff = lse_row(p, b, h, sr);
    float slope2 = 0.f;
    if constexpr (ALIBI) slope2 = p.alibi[(long)b * p.alibi_bstride + h] * kLog2e;
    if (h != hk * group) __syncthreads();  // every wave is done with the previous head's tiles

    Stream st;
    st.abase = p.q + qoff;
    st.bbase = p.dout + qoff;
    st.lo = 0;
    st.hi = Sq;
    st.row_stride = (int)rs;
    st.row_bytes = (int)rs * 2;
    st.init(wave, lane);
    // L and D of a tile.  Wave 1 loads D straight into LDS (4 bytes per lane, rows past
    // the end read as zeros).  Wave 0 loads L into a register and, once it has landed,
    // stores it to LDS in log2 units with -inf (a row that saw no key) and rows past the
    // end as +inf, so that every P of such a row is exp2(-inf) = 0: the per-score loop
    // then needs one FMA before the exponential, where scaling and testing each of its
    // 32 copies of L cost three vector instructions per score.
    auto load_d = [&](lds_u8* dst, int t) {
      if (wave == 1) {
        const int r0 = t * DKV_TILE;
        const float* src = p.delta + loff + r0;
        const int n = max(0, min(DKV_TILE, Sq - r0)) * 4;
        const auto rsr = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, n, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsr, dst + LDBYTES, 4, 4 * lane, 0, 0, 0);
      }
    };
    auto load_l = [&](int t) {  // wave 0: this lane's row of tile t
      const int r = t * DKV_TILE + lane;
      return (lane < DKV_TILE && r < Sq) ? p.lse[loff + r] : -INFINITY;
    };
    auto put_l = [&](lds_u8* dst, float l) {  // wave 0
      if (lane < DKV_TILE) ((__attribute__((address_space(3))) float*)dst)[lane] = l == -INFINITY ? INFINITY : l * kLog2e;
    };
    float lraw = -INFINITY;  // wave 0: L of this lane's row of the next tile, in flight

    if (t_begin < t_end) {
      st.load(lds, lds + GOFF, t_begin);
      load_d(lds + LOFF, t_begin);
      if (wave == 0) lraw = load_l(t_begin);
    }
    // One query tile: S, dP, then P and dS, then dV and dK.  MODE 0: no mask (every pair
    // visible); 1: with the mask (a mask boundary or the end crosses the tile); 2: which of
    // the two is decided per tile, by a branch around P and dS (headdim 256, below); 3: no
    // pair visible: only this wave's share of the loads and the barrier.
    auto step = [&](int t, auto mode) {
      constexpr int MODE = decltype(mode)::value;
      const int cur = (t - t_begin) & 1;
      wait_tile_loads<0>();
      if (wave == 0) put_l(lds + cur * BUF + LOFF, lraw);
      __syncthreads();
      if (t + 1 < t_end) {
        lds_u8* nb = lds + (cur ^ 1) * BUF;
        st.load(nb, nb + GOFF, t + 1);
        load_d(nb + LOFF, t + 1);
        if (wave == 0) lraw = load_l(t + 1);
      }
      if constexpr (MODE == 3) return;  // no query of the tile sees a key of this wave
      const lds_u8* qt = lds + cur * BUF;
      const lds_u8* gt = qt + GOFF;
      const __attribute__((address_space(3))) float* lt = (const __attribute__((address_space(3))) float*)(qt + LOFF);

      f32x16 s[DKV_QB], dp[DKV_QB];
#pragma unroll
      for (int qb = 0; qb < DKV_QB; ++qb) s[qb] = dp[qb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < HD / 16; ++kk)
#pragma unroll
        for (int qb = 0; qb < DKV_QB; ++qb) {
          s[qb] = mfma32(row_operand<QP, E>(qt, lrow, half, qb, kk), kf[kk], s[qb]);
          const x8<E> vb = VLDS ? *(const __attribute__((address_space(3))) x8<E>*)(vrow + 32 * kk) : vf[VLDS ? 0 : kk];
          dp[qb] = mfma32(row_operand<QP, E>(gt, lrow, half, qb, kk), vb, dp[qb]);
        }

      // register r of block qb holds query i0 + 32 qb + 16 (r / 8) + 8 half + r % 8 of the tile
      const int i0 = t * DKV_TILE;
      x8<E> pf[2 * DKV_QB], dsf[2 * DKV_QB];
      auto scores = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
        for (int cc = 0; cc < 2 * DKV_QB; ++cc) {
          const int qb = cc >> 1, ci = cc & 1;
          const int qrow = 16 * cc + 8 * half;  // first tile row of this chunk
          typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
          const f32x4 l_a = *(const lds_f32x4*)(lt + qrow);
          const f32x4 l_b = *(const lds_f32x4*)(lt + qrow + 4);
          const f32x4 d_a = *(const lds_f32x4*)(lt + LDBYTES / 4 + qrow);
          const f32x4 d_b = *(const lds_f32x4*)(lt + LDBYTES / 4 + qrow + 4);
          f32x16 pt, dt;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float l2 = e < 4 ? l_a[e] : l_b[e - 4];  // L in log2 units, +inf: P = 0
            const float dd = e < 4 ? d_a[e] : d_b[e - 4];
            const int qi = i0 + qrow + e;
            float x = fmaf(s[qb][8 * ci + e], c, -l2);
            if constexpr (ALIBI) x += alibi_log2(slope2, qi + off, my_k);
            float pv = fast_exp2(x);
            if constexpr (MASKED) pv = ((uint32_t)(qi - qlo) <= (uint32_t)(qhi - qlo) && qlo <= qhi) ? pv : 0.f;
            pt[e] = pv;
            dt[e] = pv * (dp[qb][8 * ci + e] - dd);
          }
          pf[cc] = pack_rows<E>(pt, 0);
          dsf[cc] = pack_rows<E>(dt, 0);
        }
      };
      if constexpr (MODE == 2) {
        const int wj0 = min(j0 + 32 * wave, Sk - 1), wjl = min(j0 + 32 * wave + 31, Sk - 1);
        const bool full = (i0 + DKV_TILE <= Sq) && (wr < 0 || i0 + off + wr >= wjl) &&
                          (wl < 0 || i0 + DKV_TILE - 1 + off - wl <= wj0);
        if (full)
          scores(std::false_type{});
        else
          scores(std::true_type{});
      } else {
        scores(std::bool_constant<MODE == 1>{});
      }

#pragma unroll
      for (int cc = 0; cc < 2 * DKV_QB; ++cc)
#pragma unroll
        for (int db = 0; db < HD / 32; ++db) {
          dv[db] = mfma32(tr_operand<QP, E>(gt, lane, db, cc), pf[cc], dv[db]);
          dk[db] = mfma32(tr_operand<QP, E>(qt, lane, db, cc), dsf[cc], dk[db]);
        }
    };
    // The tiles every (query, key of this wave) pair of which is visible, with no query
    // past the end, form one range [tf_begin, tf_end): run there without the mask, in a
    // loop of its own, so that the mask costs nothing on them and the loop body is one
    // block (an explicit branch per tile cost the products' overlap with the
    // exponentials; the compiler's own select computed the mask on every tile).  Every
    // wave passes the same number of steps, each with one barrier.
    const int wj0 = min(j0 + 32 * wave, Sk - 1), wjl = min(j0 + 32 * wave + 31, Sk - 1);
    int tf_lo = 0, tf_hi = Sq / DKV_TILE;  // full tiles: tf_lo <= t < tf_hi
    if (wr >= 0) {
      const int x = wjl - off - wr;  // needs t * DKV_TILE >= x
      tf_lo = x <= 0 ? 0 : (x + DKV_TILE - 1) / DKV_TILE;
    }
    if (wl >= 0) {
      const int y = wj0 - off + wl - DKV_TILE + 1;  // needs t * DKV_TILE <= y
      tf_hi = min(tf_hi, y < 0 ? 0 : y / DKV_TILE + 1);
    }
    // the tiles with any query that sees a key of this wave: [tv_begin, tv_end)
    const int qvlo = wr < 0 ? 0 : max(0, wj0 - off - wr), qvhi = wl < 0 ? Sq - 1 : min(Sq - 1, wjl - off + wl);
    const int tv_begin = qvhi < qvlo ? t_end : min(max(t_begin, qvlo / DKV_TILE), t_end);
    const int tv_end = qvhi < qvlo ? t_end : max(tv_begin, min(t_end, qvhi / DKV_TILE + 1));
    const int tf_begin = min(max(tv_begin, tf_lo), tv_end);
    const int tf_end = max(tf_begin, min(tv_end, tf_hi));
    // (at headdim 256 the three loops cost the kernel a third more time: its registers
    // are full, and the compiler copied the accumulators between the loops; one loop with
    // the branch around P and dS there)
    if constexpr (HD == 256) {
      for (int t = t_begin; t < t_end; ++t) step(t, std::integral_constant<int, 2>{});
    } else {
      int t = t_begin;
      for (; t < tv_begin; ++t) step(t, std::integral_constant<int, 3>{});
      for (; t < tf_begin; ++t) step(t, std::integral_constant<int, 1>{});
      for (; t < tf_end; ++t) step(t, std::integral_constant<int, 0>{});
      for (; t < tv_end; ++t) step(t, std::integral_constant<int, 1>{});
      for (; t < t_end; ++t) step(t, std::integral_constant<int, 3>{});
    }
  }  // query heads of the group
  if (my_k < Sk) {
    store_rows<HD, E>(p.dk + koff, rsk, my_k, dk, p.scale, half);
    store_rows<HD, E>(p.dv + koff, rsk, my_k, dv, 1.f, half);
  }
#endif
}

hipError_t launch_bwd(const BwdParams& p, int headdim, hipStream_t stream);
// dq_kernel launches (fa_bwd_dq.hip: its own register-allocation flags)
hipError_t launch_dq_d64(const BwdParams& p, hipStream_t stream);
hipError_t launch_dq_d128(const BwdParams& p, hipStream_t stream);

template <int HD, typename E>
hipError_t launch_dq_hd(const BwdParams& p, hipStream_t stream) {
  const int items = p.batch * p.nheads * p.num_q_tiles;
  if (p.alibi != nullptr)
    hipLaunchKernelGGL((dq_kernel<HD, true, E>), dim3(items), dim3(256), 0, stream, p, items);
  else
    hipLaunchKernelGGL((dq_kernel<HD, false, E>), dim3(items), dim3(256), 0, stream, p, items);
  return hipGetLastError();
}

}  // namespace fa
