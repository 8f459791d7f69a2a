// fa_fwd_kernel.h - matrix-core (MFMA) attention forward for gfx950 (kernel templates;
// fa_fwd_d{64,128,256}.hip instantiate them, fa_fwd_launch.hip dispatches).
//
// What it computes: for each (batch, head) and query row i,
//   out_i = sum_j softmax_j(scale * q_i.k_j + bias_ij) v_j   over the visible keys j,
//   lse_i = ln sum_j exp(scale * q_i.k_j + bias_ij),
// following the page "FlashAttention：快速且内存高效的准确注意力机制"
// (cloud.tencent.com.cn/developer/article/2433927), sections "使用示例" and "参数说明"
// (the computation and its arguments), "算法 / 前向传播" (blocked over query rows,
// unscaled running output with one final division by the row sum, logsumexp as
// the second output), "并行性" (grid over batch x heads, plus the sequence
// dimension for long inputs), "工作分区" (query rows split across the waves of a
// block, K and V shared by all of them), "2.1" (bottom-right causal alignment,
// zero rows) and "2.3" (sliding window).
//
// Design for CDNA4 (not a translation of the pages' A100 layout):
//  * one workgroup = 4 wave64s = 128 query rows (32 per wave); one workgroup per
//    (batch, head, query tile[, key split]); the linear block id is remapped so
//    that each XCD works on a contiguous range of (batch, head) and keeps that
//    head's K/V in its own L2;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    every lane owns one query column, so the softmax row statistics are
//    lane-local plus one v_permlane32_swap between the two half-waves;
//  * K rows are stored in LDS with bits 2 and 3 of the row index swapped; with
//    that order the fp32 S^T accumulator, rounded to bf16, is already laid out as
//    the B operand of O^T += V^T P^T, so P never leaves the registers;
//  * V is transposed once, in registers, on its way into LDS (V^T rows of 64 keys)
//    so the A operand of O^T += V^T P^T is a plain 16-byte LDS read;
//  * two-stage software pipeline per 64-key tile t: the products for S(t+1) are
//    issued between the exponentials of tile t, and O += V(t) P(t) between the
//    row maxima of S(t+1), so the matrix cores and the vector ALUs work together;
//    K runs two tiles ahead of the compute and V one tile ahead, double buffered
//    in LDS, one barrier per tile;
//  * the running maximum is only moved (and O, l rescaled) when a row's maximum
//    grows by more than 2^8; otherwise the stale maximum is kept, which leaves the
//    result exact (O and l share it) and removes the rescale from almost every tile;
//  * exponentials use exp2 with scale*log2(e) folded into one FMA; the row sum is
//    accumulated from the fp32 exponentials (P is rounded to bf16 only for P V);
//  * K/V tiles are read with buffer loads whose range ends at the last valid key,
//    so ragged tails read zeros without branches; only tiles crossing a mask
//    boundary run the per-element visibility test.
#pragma once
#include "fa_common.h"

namespace fa {

constexpr int BR = 128;        // query rows per workgroup
constexpr int BC = 64;         // keys per tile
constexpr int NTHREADS = 256;  // 4 waves
constexpr int PAD = 8;         // bf16 padding per LDS row (16 bytes) against bank conflicts
constexpr float RESCALE_TH = 8.0f;  // log2 units: keep a stale max while p <= 2^8

template <int HD>
struct Tile {
  static constexpr int KROW = HD + PAD;   // K tile row pitch in LDS (elements)
  static constexpr int VROW = BC + PAD;   // V^T tile row pitch in LDS (elements)
  static constexpr int KELEMS = BC * KROW;
  static constexpr int VELEMS = HD * VROW;
  static constexpr int LDS_ELEMS = 2 * (KELEMS + VELEMS);  // two buffers each
  static constexpr int CPR = HD / 8;      // 16-byte chunks per K/V row
  static constexpr int KU = BC * CPR / NTHREADS;  // K chunks per thread (= HD/32)
  static constexpr int KR = HD / 32;      // V rows per thread (one 8-wide column chunk)
  static constexpr int KB = BC / KR;      // V key blocks across the tile
};

// LDS row that holds key `row` of the tile: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int k_lds_row(int row) {
  return (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);
}

// Buffer resource over `rows` rows of a K or V tile starting at `base`; loads past
// the last row return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int rows, int row_bytes) {
  const int n = rows > 0 ? min(rows, BC) * row_bytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
}

// Two bf16 halves (`half` 0 = low, 1 = high) of a and b, packed a-first.
__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, int half) {
  return half == 0 ? ((a & 0xffffu) | (b << 16)) : ((a >> 16) | (b & 0xffff0000u));
}

template <int HD>
__device__ __forceinline__ void store_k(const u32x4 (&kr)[Tile<HD>::KU], uint16_t* ks, int tid) {
  using T = Tile<HD>;
#pragma unroll
  for (int u = 0; u < T::KU; ++u) {
    const int id = tid + NTHREADS * u;
    const int row = id / T::CPR, col = id % T::CPR;
    *(u32x4*)(ks + k_lds_row(row) * T::KROW + col * 8) = kr[u];
  }
}

// V^T: this thread holds KR consecutive keys x 8 consecutive columns; write each
// column as KR consecutive keys of one V^T row.
template <int HD>
__device__ __forceinline__ void store_vt(const u32x4 (&vr)[Tile<HD>::KR], uint16_t* vt, int tid) {
  using T = Tile<HD>;
  const int kb = tid % T::KB, dc = tid / T::KB;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint16_t* dst = vt + (dc * 8 + d) * T::VROW + kb * T::KR;
    const int w = d >> 1, hf = d & 1;
    if constexpr (T::KR == 2) {
      *(uint32_t*)dst = pick_pair(vr[0][w], vr[1][w], hf);
    } else if constexpr (T::KR == 4) {
      u32x2 o = {pick_pair(vr[0][w], vr[1][w], hf), pick_pair(vr[2][w], vr[3][w], hf)};
      *(u32x2*)dst = o;
    } else {
      u32x4 o = {pick_pair(vr[0][w], vr[1][w], hf), pick_pair(vr[2][w], vr[3][w], hf),
                 pick_pair(vr[4][w], vr[5][w], hf), pick_pair(vr[6][w], vr[7][w], hf)};
      *(u32x4*)dst = o;
    }
  }
}

template <int HD>
struct KVStream {
  using T = Tile<HD>;
  const uint16_t* kbase;
  const uint16_t* vbase;
  int key_lo, key_hi, row_bytes;
  int row_stride;          // elements between consecutive keys
  uint32_t k_off[T::KU];   // byte offsets of this thread's K chunks inside a tile
  uint32_t v_off[T::KR];   // byte offsets of this thread's V rows inside a tile

  __device__ __forceinline__ void init(int tid) {
#pragma unroll
    for (int u = 0; u < T::KU; ++u) {
      const int id = tid + NTHREADS * u;
      k_off[u] = (uint32_t)((id / T::CPR) * row_bytes + (id % T::CPR) * 16);
    }
    const int kb = tid % T::KB, dc = tid / T::KB;
#pragma unroll
    for (int rr = 0; rr < T::KR; ++rr) v_off[rr] = (uint32_t)((kb * T::KR + rr) * row_bytes + dc * 16);
  }
  // tile t starts at key key_lo + t*BC; keys at or past key_hi read as zeros
  __device__ __forceinline__ void load_k(u32x4 (&kr)[T::KU], int t) const {
    const int j0 = key_lo + t * BC;
    const auto rs = tile_rsrc(kbase + (long)j0 * row_stride, key_hi - j0, row_bytes);
#pragma unroll
    for (int u = 0; u < T::KU; ++u)
      kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)k_off[u], 0, 0));
  }
  __device__ __forceinline__ void load_v(u32x4 (&vr)[T::KR], int t) const {
    const int j0 = key_lo + t * BC;
    const auto rs = tile_rsrc(vbase + (long)j0 * row_stride, key_hi - j0, row_bytes);
#pragma unroll
    for (int rr = 0; rr < T::KR; ++rr)
      vr[rr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)v_off[rr], 0, 0));
  }
};

// S^T (64 keys x 32 queries of this wave) = K_tile Q^T, two 32x32 blocks.
template <int HD>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const uint16_t* kt, const bf16x8 (&qf)[HD / 16],
                                        int lrow, int half) {
  using T = Tile<HD>;
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < HD / 16; ++kk) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a = *(const bf16x8*)(kt + (32 * kb + lrow) * T::KROW + 16 * kk + 8 * half);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
    }
  }
}

// ALiBi: turn the raw scores of one tile into log2 units with the bias added,
// scale*log2e*s - slope*log2e*|pos - key|.  Without ALiBi the scores stay raw.
__device__ __forceinline__ void bias_tile(f32x16 (&s)[2], int j0, int my_pos, float c, float slope, int half) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // key held by (lane, r): see k_lds_row for the row order
      const int key = j0 + 32 * kb + 16 * (r >> 3) + 8 * half + (r & 7);
      s[kb][r] = s[kb][r] * c - slope * fabsf((float)(my_pos - key));
    }
  }
}

// Set the scores of keys this row may not see to -inf (tiles crossing a mask boundary).
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int j0, int key_hi, int my_pos, int wl, int wr, int half) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + 32 * kb + 16 * (r >> 3) + 8 * half + (r & 7);
      const bool vis = key < key_hi && (wl < 0 || key >= my_pos - wl) && (wr < 0 || key <= my_pos + wr);
      s[kb][r] = vis ? s[kb][r] : -INFINITY;
    }
  }
}

// Max of the scores in log2 units: the stored max times `cs` (> 0); -inf stays -inf.
__device__ __forceinline__ float to_log2(float mx, float cs) { return mx == -INFINITY ? mx : mx * cs; }

__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
  float m0 = fmaxf(s[0][0], s[0][1]);
  float m1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) {
    m0 = fmaxf(m0, fmaxf(s[0][r], s[0][r + 1]));
    m1 = fmaxf(m1, fmaxf(s[1][r], s[1][r + 1]));
  }
  return max_with_other_half(fmaxf(m0, m1));
}

// Instruction-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200;

// Per-wave state of the forward loop.
template <int HD>
struct FwdState {
  bf16x8 qf[HD / 16];       // Q^T fragments (B operand of S^T = K Q^T)
  f32x16 oacc[HD / 32];     // O^T accumulator, unscaled
  float m_run;              // reference maximum of the exponentials (log2 units)
  float l_run;              // this lane's share of the row sum against m_run
};

// One tile step: P(t) from s_cur, S(t+1) into s_nxt, O += V(t) P(t), staging of
// K(t+2) and V(t+1), reference-maximum update.  Ends with the tile barrier.
template <int HD, bool ALIBI>
__device__ __forceinline__ void tile_step(FwdState<HD>& st, const f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], int t,
                                          int t_begin, const KVStream<HD>& kv, uint16_t* ks0, uint16_t* vt0,
                                          u32x4 (&kreg)[Tile<HD>::KU], u32x4 (&vreg)[Tile<HD>::KR], int tid,
                                          int lrow, int half, float c, float cs, float slope, int my_pos,
                                          int wl, int wr, int i0, int i_last, int off) {
  using T = Tile<HD>;
  const int par = (t - t_begin) & 1;
  const uint16_t* const k_next = ks0 + (par ^ 1) * T::KELEMS;  // K of tile t+1
  uint16_t* const k_free = ks0 + par * T::KELEMS;              // receives K of tile t+2
  const uint16_t* const v_cur = vt0 + par * T::VELEMS;         // V of tile t
  uint16_t* const v_free = vt0 + (par ^ 1) * T::VELEMS;        // receives V of tile t+1

  kv.load_k(kreg, t + 2);  // past the last tile these read zeros or unused keys: harmless
  kv.load_v(vreg, t + 1);

  // S(t+1) = K(t+1) Q^T
  qk_tile<HD>(s_nxt, k_next, st.qf, lrow, half);

  // P(t) = exp2(S(t) * cs - m), rounded to bf16 for the P V product
  const float negm = (st.m_run == -INFINITY) ? 0.f : -st.m_run;
  bf16x8 pf[4];
  float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
    const int kb = ci >> 1, r0 = 8 * (ci & 1);
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(fmaf(s_cur[kb][r0 + 2 * e], cs, negm));
      const float p1 = fast_exp2(fmaf(s_cur[kb][r0 + 2 * e + 1], cs, negm));
      pk[e] = pack_bf16x2(p0, p1);
      // the row sum stays in fp32: the lse needs it to ~1e-4 relative, which a sum
      // of bf16-rounded terms (2^-9 each) cannot guarantee
      lsum0 += p0;
      lsum1 += p1;
    }
    pf[ci] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
  }
  st.l_run += lsum0 + lsum1;

  // O^T += V(t)^T P(t)^T
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) {
      const bf16x8 a = *(const bf16x8*)(v_cur + (32 * db + lrow) * T::VROW + 16 * ci + 8 * half);
      st.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ci], st.oacc[db], 0, 0, 0);
    }
  }

  // max of S(t+1) before masking: exact for tiles every row sees in full
  const int j1 = kv.key_lo + (t + 1) * BC;
  if constexpr (ALIBI) bias_tile(s_nxt, j1, my_pos, c, slope, half);
  float mx = tile_max(s_nxt);

  store_k<HD>(kreg, k_free, tid);
  store_vt<HD>(vreg, v_free, tid);

  // Issue order: loads first, then S(t+1) products spread through the exponentials,
  // then the P V products spread through the max of S(t+1) and the LDS stores.
  __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, Tile<HD>::KU + Tile<HD>::KR, 0);
#pragma unroll
  for (int i = 0; i < HD / 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
  }
#pragma unroll
  for (int i = 0; i < HD / 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
  }

  // tiles crossing a mask boundary: mask, then take the max again
  const bool nxt_full = (j1 + BC <= kv.key_hi) && (wl < 0 || j1 >= i_last + off - wl) &&
                        (wr < 0 || j1 + BC - 1 <= i0 + off + wr);
  if (!nxt_full) {
    mask_tile(s_nxt, j1, kv.key_hi, my_pos, wl, wr, half);
    mx = tile_max(s_nxt);
  }

  // move the reference maximum only when a row grew by more than 2^8
  const float m_new = fmaxf(st.m_run, to_log2(mx, cs));
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(m_new > st.m_run + RESCALE_TH) != 0, 0)) {
    // 0 when only m_run is -inf; 1 for a row that has seen no visible key yet
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
    st.m_run = m_new;
  }
  __syncthreads();
}

template <int HD, bool ALIBI, bool SPLIT>
__global__ __launch_bounds__(NTHREADS) void fwd_kernel(FwdParams p) {
  using T = Tile<HD>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[T::LDS_ELEMS];
  uint16_t* const ks0 = smem;
  uint16_t* const vt0 = smem + 2 * T::KELEMS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;  // query column / A-operand row owned by this lane
  const int half = lane >> 5;  // which 8-element k slice this lane feeds

  // ---- work item -------------------------------------------------------------
  int w = xcd_remap(blockIdx.x, gridDim.x);
  int qt = w % p.num_q_tiles;
  w /= p.num_q_tiles;
  int split = 0;
  if constexpr (SPLIT) {
    split = w % p.num_splits;
    w /= p.num_splits;
  }
  const int h = w % p.nheads;
  const int b = w / p.nheads;
  if (p.reverse_q) qt = p.num_q_tiles - 1 - qt;

  const int Sq = p.seqlen_q, Sk = p.seqlen_k;
  int key_lo = 0, key_hi = Sk;
  if constexpr (SPLIT) {
    key_lo = min(Sk, split * p.split_len);
    key_hi = min(Sk, key_lo + p.split_len);
  }
  const long row_stride = (long)p.nheads * HD;
  const uint16_t* __restrict__ qbase = p.q + (long)b * Sq * row_stride + (long)h * HD;

  KVStream<HD> kv;
  kv.kbase = p.k + (long)b * Sk * row_stride + (long)h * HD;
  kv.vbase = p.v + (long)b * Sk * row_stride + (long)h * HD;
  kv.key_lo = key_lo;
  kv.key_hi = key_hi;
  kv.row_stride = (int)row_stride;
  kv.row_bytes = (int)row_stride * 2;
  kv.init(tid);

  const int i0 = qt * BR;
  const int i_last = min(i0 + BR, Sq) - 1;
  const int off = Sk - Sq;  // query i sits at key position i + off
  const int wl = p.window_left, wr = p.window_right;

  // Key tiles that any row of this block can see.
  int lo = key_lo, hi = key_hi - 1;
  if (wl >= 0) lo = max(lo, i0 + off - wl);
  if (wr >= 0) hi = min(hi, i_last + off + wr);
  int t_begin = 0, t_end = 0;
  if (hi >= lo) {
    t_begin = (lo - key_lo) / BC;
    t_end = (hi - key_lo) / BC + 1;
  }

  // ---- Q fragments: B operand of S^T = K Q^T, held for the whole loop ----------
  FwdState<HD> st;
  const int my_q = i0 + wave * 32 + lrow;
  const int my_pos = my_q + off;
#pragma unroll
  for (int kk = 0; kk < HD / 16; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_q < Sq) raw = *(const u32x4*)(qbase + (long)my_q * row_stride + 16 * kk + 8 * half);
    raw = (raw & p.q_and) ^ p.q_sign;
    st.qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }
#pragma unroll
  for (int db = 0; db < HD / 32; ++db) st.oacc[db] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  const float c = p.scale_log2;
  float slope = 0.f;
  if constexpr (ALIBI) slope = p.alibi[h] * kLog2e;  // bias in log2 units
  // multiplier turning the stored scores into log2 units
  const float cs = ALIBI ? 1.f : c;

  f32x16 s_a[2], s_b[2];
  u32x4 kreg[T::KU], vreg[T::KR];

  if (t_begin < t_end) {
    // prologue: K and V of the first tile, K of the second, then S of the first
    kv.load_k(kreg, t_begin);
    kv.load_v(vreg, t_begin);
    store_k<HD>(kreg, ks0, tid);
    store_vt<HD>(vreg, vt0, tid);
    kv.load_k(kreg, t_begin + 1);  // zeros when past the last key: harmless
    store_k<HD>(kreg, ks0 + T::KELEMS, tid);
    __syncthreads();
    qk_tile<HD>(s_a, ks0, st.qf, lrow, half);
    const int j0 = key_lo + t_begin * BC;
    if constexpr (ALIBI) bias_tile(s_a, j0, my_pos, c, slope, half);
    mask_tile(s_a, j0, key_hi, my_pos, wl, wr, half);
    st.m_run = to_log2(tile_max(s_a), cs);
    __syncthreads();  // every wave is done with K(t_begin) before the loop refills its buffer
  }

  // two tiles per trip so S(t) and S(t+1) swap roles without register copies
  for (int t = t_begin; t < t_end; t += 2) {
    tile_step<HD, ALIBI>(st, s_a, s_b, t, t_begin, kv, ks0, vt0, kreg, vreg, tid, lrow, half, c, cs, slope,
                         my_pos, wl, wr, i0, i_last, off);
    if (t + 1 >= t_end) break;
    tile_step<HD, ALIBI>(st, s_b, s_a, t + 1, t_begin, kv, ks0, vt0, kreg, vreg, tid, lrow, half, c, cs,
                         slope, my_pos, wl, wr, i0, i_last, off);
  }
  f32x16* const oacc = st.oacc;
  const float m_run = st.m_run;
  const float l_run = st.l_run;

  // ---- epilogue: one division per row, logsumexp ------------------------------
  const float l_tot = sum_with_other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
  if (my_q >= Sq) return;

  if constexpr (!SPLIT) {
    uint16_t* obase = (uint16_t*)p.out + ((long)b * Sq + my_q) * row_stride + (long)h * HD;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // accumulator rows 4g..4g+3 of block db hold columns 32db + 8g + 4*half + 0..3
        const int d0 = 32 * db + 8 * g + 4 * half;
        u32x2 o = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                   pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *(u32x2*)(obase + d0) = o;
      }
    if (half == 0) p.lse[((long)b * p.nheads + h) * Sq + my_q] = lse_v;
  } else {
    const long rowid = (((long)split * p.batch + b) * p.nheads + h) * Sq + my_q;
    float* obase = (float*)p.out + rowid * HD;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * half;
        f32x4 o = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                   oacc[db][4 * g + 3] * inv};
        *(f32x4*)(obase + d0) = o;
      }
    if (half == 0) p.lse[rowid] = lse_v;
  }
}

template <int HD, bool ALIBI, bool SPLIT>
hipError_t launch_fwd_instance(const FwdParams& p, long nblocks, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<HD, ALIBI, SPLIT>), dim3((unsigned)nblocks), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

// One translation unit per head dimension instantiates these (separate files let
// each get its own register-allocation flags).
template <int HD>
hipError_t launch_fwd_hd(const FwdParams& p, bool split, hipStream_t stream) {
  const long nblocks = (long)p.batch * p.nheads * p.num_q_tiles * (split ? p.num_splits : 1);
  const bool alibi = p.alibi != nullptr;
  if (split) return alibi ? launch_fwd_instance<HD, true, true>(p, nblocks, stream)
                          : launch_fwd_instance<HD, false, true>(p, nblocks, stream);
  return alibi ? launch_fwd_instance<HD, true, false>(p, nblocks, stream)
               : launch_fwd_instance<HD, false, false>(p, nblocks, stream);
}

hipError_t launch_fwd_d64(const FwdParams& p, bool split, hipStream_t stream);
hipError_t launch_fwd_d128(const FwdParams& p, bool split, hipStream_t stream);
hipError_t launch_fwd_d256(const FwdParams& p, bool split, hipStream_t stream);

}  // namespace fa
