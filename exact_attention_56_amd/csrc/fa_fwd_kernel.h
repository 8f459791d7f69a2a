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
// zero rows), "2.3" (sliding window) and "2.4" (ALiBi).  q/k/v/out are bf16 or
// fp16 (the element type E); the arithmetic is the same for both.
//
// Design for CDNA4 (not a translation of the pages' A100 layout):
//  * one workgroup = 4 wave64s = 128 query rows (32 per wave); one workgroup per
//    (batch, head, query tile[, key split]); the linear block id is remapped so
//    that each XCD works on a contiguous range of (batch, head) and keeps that
//    head's K/V in its own L2;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16/f16:
//    every lane owns one query column, so the softmax row statistics are
//    lane-local plus one v_permlane32_swap between the two half-waves;
//  * K rows are stored in LDS with bits 2 and 3 of the row index swapped; with
//    that order the fp32 S^T accumulator, rounded to 16 bits, is already laid out as
//    the B operand of O^T += V^T P^T, so P never leaves the registers;
//  * K and V tiles go from HBM straight into LDS (buffer loads with the LDS
//    destination, no staging registers); V stays in its natural [key][d] layout
//    and the A operand of O^T += V^T P^T is assembled with two ds_read_b64_tr_b16
//    transpose reads per product;
//  * two-stage software pipeline per 64-key tile t: the products for S(t+1) are
//    issued between the exponentials of tile t, and O += V(t) P(t) between the
//    row maxima of S(t+1), so the matrix cores and the vector ALUs work together;
//    K runs two tiles ahead of the compute and V one tile ahead, double buffered
//    in LDS, one barrier per tile;
//  * the running maximum is only moved (and O, l rescaled) when a row's maximum
//    grows by more than 2^8; otherwise the stale maximum is kept, which leaves the
//    result exact (O and l share it) and removes the rescale from almost every tile;
//  * exponentials use exp2 with scale*log2(e) folded into one FMA; the row sum is
//    accumulated from the fp32 exponentials (P is rounded to E only for P V);
//  * the buffer loads' range ends at the last valid key, so ragged tails land in
//    LDS as zeros without branches; only tiles crossing a mask boundary run the
//    per-element visibility test.
#pragma once
#include <type_traits>

#include "fa_common.h"

namespace fa {

// A workgroup has NW = 4 or 8 waves of 32 query rows each.  Eight waves (256 rows,
// the ping-pong schedule below) halve the K/V traffic from L2 per flop; headdim 128
// uses them where they measured faster (fwd_waves), everything else four.
constexpr int BC = 64;  // keys per tile
constexpr float RESCALE_TH = 8.0f;  // log2 units: keep a stale max while p <= 2^8
// Kernels without ALiBi (headdim 64 and 128) keep the reference maximum without a
// per-tile row max (refit_reference); 0 takes the row max of every tile instead.
#ifndef FA_NOMAX
#define FA_NOMAX 1
#endif
constexpr uint32_t OOB_OFFSET = 0x80000000u;  // buffer offset past any tile: reads as zero
// The ALiBi kernels with the keys right to left (causal; headdim 64 and 128) add the
// linear bias on the matrix cores: the K rows' pad slots hold each row's key index and
// the Q side a split of the bias step (qk_tile); the loads then leave the pad slots alone.
#ifndef FA_ALIBI_AUG
#define FA_ALIBI_AUG 1
#endif
constexpr uint32_t PAD_KEEP = 0xffffffffu;  // K slot offset: a pad slot the loads skip

// LDS tiles.  A K row keeps its HD/8 16-byte chunks plus one pad slot (16 lanes
// reading one chunk column of 16 rows then hit 16 distinct 4-bank groups); the pad
// slot is filled with zeros by an out-of-range load (or, in the causal ALiBi kernels,
// holds the row's key index for the bias product, see qk_tile).  V is stored in 64-byte column
// blocks: block db holds columns 32db..32db+31 of the tile's 64 rows, 64 bytes per row,
// so the 32 lanes that one half of a transpose read serves (4 rows x 32 columns) read
// 256 contiguous bytes, all 64 banks once, and the tile needs no pad slot.  (Padded
// rows of HD + 16 columns left a 2-way conflict on every transpose read; HD + 32
// removed it but its two extra loads per tile cost more than the conflicts.)
template <int HD, int NW>
struct Tile {
  static_assert(NW == 4 || NW == 8, "four or eight waves per workgroup");
  static constexpr int CPR = HD / 8;         // 16-byte chunks per K/V row in memory
  static constexpr int KCH = CPR + 1;        // 16-byte slots per K row in LDS
#ifndef FA_VBLOCK
#define FA_VBLOCK 1
#endif
  // V: with FA_VBLOCK the tile is stored in 64-byte column blocks, [HD / 32][BC rows][4
  // chunks] (no pad slots, CPR loads per tile); otherwise in padded rows of VCH slots
  static constexpr int VCH = FA_VBLOCK ? CPR : CPR + 2;  // 1 KiB loads per V tile
  static constexpr int KPITCH = KCH * 16;    // bytes
  static constexpr int VPITCH = FA_VBLOCK ? 64 : VCH * 16;  // bytes between V rows (within a block)
  static constexpr int VBLOCK = FA_VBLOCK ? BC * 64 : 64;   // bytes between 32-column blocks of V
  // 64-lane (1 KiB) direct loads per tile: the tile needs KCH (VCH) of them, load u
  // issued by loading wave u % 4.  A wave skips the loads that would lie wholly past
  // the tile (a wave-uniform test): issuing them as all-zero loads, so that every
  // wave issued the same number, cost measurably (20 instead of 17 K loads per tile
  // at headdim 128).
  static constexpr int KPW = (KCH + 3) / 4;  // most K loads a loading wave issues (4 waves load K)
  static constexpr int VPW = (VCH + 3) / 4;  // most V loads a loading wave issues (4 waves load V)
  static constexpr int KBYTES = 1024 * KCH;  // one K buffer (>= BC * KPITCH)
  static constexpr int VBYTES = 1024 * VCH;  // one V buffer (>= BC * VPITCH)
  // Ring of NBUF K and NBUF V buffers: K runs NBUF tiles ahead of the step that
  // reads it and V NBUF-1, so a tile's loads have NBUF-1 steps to land.  Headdim 64
  // measured slower with three buffers, so every headdim keeps two.
#ifndef FA_NBUF
#define FA_NBUF 2
#endif
  static constexpr int NBUF = HD == 256 ? 2 : FA_NBUF;
  static constexpr int LDS_BYTES = NBUF * (KBYTES + VBYTES);
  // most loads a wave issues per step (the size of the scheduling group), and the
  // fewest: a wait until at most MIN_LOADS_PER_STEP of its loads are in flight
  // leaves every earlier step's loads landed
  static constexpr int LOADS_PER_STEP = NW == 4 ? KPW + VPW : KPW;
  static constexpr int MIN_LOADS_PER_STEP = NW == 4 ? KCH / 4 + VCH / 4 : (KCH < VCH ? KCH : VCH) / 4;
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed LDS read (ds_read_b64_tr_b16) of 4 16-bit values.  The kernels order their
// direct-to-LDS tile loads and the reads of a tile themselves (vmcnt wait, then barrier,
// and a load only ever targets a buffer no wave is reading).  Through a plain pointer
// the compiler cannot tell which buffer the read touches and makes it wait for every
// such load in flight, the next tile's included; the restrict-qualified pointer gives
// the read alias information, as ordinary LDS loads have, and drops that wait.
#ifndef FA_TR_RESTRICT
#define FA_TR_RESTRICT 1
#endif
#if FA_TR_RESTRICT
__device__ __forceinline__ s16x4 lds_read_tr(const lds_u8* __restrict__ p) {
#else
__device__ __forceinline__ s16x4 lds_read_tr(const lds_u8* p) {
#endif
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

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

// Streams K and V tiles from HBM into LDS.  Load u of a tile (wave u % 4 issues
// it) fills LDS bytes [1024u, 1024u + 1024) of the buffer, lane l the 16-byte
// slot 64u + l, i.e. row (64u + l) / KCH, slot (64u + l) % KCH; the lane fetches
// the matching 16 bytes (K rows in the k_lds_row order) or, for a pad slot or a
// slot past the last row, an out-of-range offset that writes zeros.
// REV: the loop's step t visits key tile t_begin + t_end - 1 - t (keys right to left);
// steps past the last (prefetches) read nothing.
template <int HD, int NW, bool REV_ = false>
struct KVStream {
  using T = Tile<HD, NW>;
  static constexpr bool REV = REV_;
  // the pad slots hold key indices (not at headdim 256: its one-wave-per-SIMD kernel ran
  // 15% slower with the two extra products, against +5% on the local ALiBi workload)
  static constexpr bool KEEP_PAD = REV && FA_ALIBI_AUG && HD != 256;
  const uint16_t* kbase;
  const uint16_t* vbase;
  int key_lo, key_hi, row_bytes;
  int t_sum, t_stop;     // REV: t_begin + t_end - 1 and t_end
  int row_stride;        // elements between consecutive keys
  int lw;                // this wave's index among the 4 waves loading a tensor
  bool loads_k, loads_v; // with 8 waves, waves 0-3 load K and waves 4-7 load V
  uint32_t koff[T::KPW]; // this lane's byte offsets inside a K tile, per load it issues
  uint32_t voff[T::VPW];

  __device__ __forceinline__ void init(int wave, int lane) {
    lw = wave & 3;
    loads_k = NW == 4 || wave < 4;
    loads_v = NW == 4 || wave >= 4;
#pragma unroll
    for (int i = 0; i < T::KPW; ++i) {
      const int slot = 64 * (lw + 4 * i) + lane;
      const int row = slot / T::KCH, ch = slot % T::KCH;
      koff[i] = (row < BC && ch < T::CPR) ? (uint32_t)(k_lds_row(row) * row_bytes + ch * 16)
                : (KEEP_PAD && row < BC) ? PAD_KEEP : OOB_OFFSET;
    }
#pragma unroll
    for (int i = 0; i < T::VPW; ++i) {
      const int slot = 64 * (lw + 4 * i) + lane;
      if constexpr (FA_VBLOCK) {
        // slot = (block * BC + row) * 4 + x holds chunk 4 * block + x of the row
        const int blk = slot / (4 * BC), row = (slot / 4) % BC, x = slot % 4;
        voff[i] = blk < T::CPR / 4 ? (uint32_t)(row * row_bytes + (4 * blk + x) * 16) : OOB_OFFSET;
      } else {
        const int row = slot / T::VCH, ch = slot % T::VCH;
        voff[i] = (row < BC && ch < T::CPR) ? (uint32_t)(row * row_bytes + ch * 16) : OOB_OFFSET;
      }
    }
  }
  // First key of the tile that step t visits: key_lo + t*BC (REV: in reverse order).
  __device__ __forceinline__ int tile_key(int t) const {
    if constexpr (REV) return key_lo + (t_sum - t) * BC;
    return key_lo + t * BC;
  }
  __device__ __forceinline__ void load_k(lds_u8* dst, int t) const {
    if (!loads_k) return;
    // keys at or past key_hi, and a REV step past the last, land as zeros
    const bool none = REV && t >= t_stop;
    const int j0 = none ? key_lo : tile_key(t);
    const auto rs = tile_rsrc(kbase + (long)j0 * row_stride, none ? 0 : key_hi - j0, row_bytes);
#pragma unroll
    for (int i = 0; i < T::KPW; ++i)
      if (lw + 4 * i < T::KCH) {
        // (a lane of a skipped pad slot writes nothing: direct loads place each lane's
        // 16 bytes by its lane index)
        if (!KEEP_PAD || koff[i] != PAD_KEEP)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + 1024 * (lw + 4 * i), 16, (int)koff[i], 0, 0, 0);
      }
  }
  __device__ __forceinline__ void load_v(lds_u8* dst, int t) const {
    if (!loads_v) return;
    // keys at or past key_hi, and a REV step past the last, land as zeros
    const bool none = REV && t >= t_stop;
    const int j0 = none ? key_lo : tile_key(t);
    const auto rs = tile_rsrc(vbase + (long)j0 * row_stride, none ? 0 : key_hi - j0, row_bytes);
#pragma unroll
    for (int i = 0; i < T::VPW; ++i)
      if (lw + 4 * i < T::VCH)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + 1024 * (lw + 4 * i), 16, (int)voff[i], 0, 0, 0);
  }
};

// KV-cache decode: the same stream over a cache whose rows are reached through a block
// table (btab == nullptr: a contiguous cache, rows in order).  Key j of the sequence is
// row (btab[j >> page_shift] << page_shift) + (j & (page_size - 1)); tiles start on
// multiples of BC <= page_size, so a tile never crosses a block.
template <int HD, int NW>
struct PagedKVStream : KVStream<HD, NW> {
  using T = Tile<HD, NW>;
  const int* btab;
  int page_shift;
  bool active;  // wave-uniform: this wave holds at least one existing row

  __device__ __forceinline__ long tile_row(int j0) const {
    if (btab == nullptr) return j0;
    // past the last key nothing is read: any block will do (and the table may end there)
    return j0 < this->key_hi ? ((long)btab[j0 >> page_shift] << page_shift) + (j0 & ((1 << page_shift) - 1)) : 0;
  }
  __device__ __forceinline__ void load_k(lds_u8* dst, int t) const {
    if (!this->loads_k) return;
    const int j0 = this->key_lo + t * BC;
    const auto rs = tile_rsrc(this->kbase + tile_row(j0) * this->row_stride, this->key_hi - j0, this->row_bytes);
#pragma unroll
    for (int i = 0; i < T::KPW; ++i)
      if (this->lw + 4 * i < T::KCH)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + 1024 * (this->lw + 4 * i), 16, (int)this->koff[i], 0, 0, 0);
  }
  __device__ __forceinline__ void load_v(lds_u8* dst, int t) const {
    if (!this->loads_v) return;
    const int j0 = this->key_lo + t * BC;
    const auto rs = tile_rsrc(this->vbase + tile_row(j0) * this->row_stride, this->key_hi - j0, this->row_bytes);
#pragma unroll
    for (int i = 0; i < T::VPW; ++i)
      if (this->lw + 4 * i < T::VCH)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + 1024 * (this->lw + 4 * i), 16, (int)this->voff[i], 0, 0, 0);
  }
};

// Wait until at most N of this wave's direct-to-LDS loads are still in flight
// (s_waitcnt vmcnt(N): low 4 bits of the count in [3:0], high 2 in [15:14]).
template <int N>
__device__ __forceinline__ void wait_tile_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// S^T (64 keys x 32 queries of this wave) = K_tile Q^T, two 32x32 blocks.
// `kt` points at this lane's row lrow, 16-byte slot `half`, of a K buffer.
// AUG: one more product per block adds g * (key index in the tile) to every score: A is
// the rows' pad slots (key index k three times, then zeros), B this lane's `baug` (g in
// three bf16 parts, half-wave 0; zeros in half-wave 1), at byte offset aug_off from kt.
// The bias product is bf16 whatever E is: with fp16 a large g (a steep slope over a small
// softmax scale) would overflow, bf16 has fp32's range.
template <int HD, typename E, bool AUG = false>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const lds_u8* kt, const x8<E> (&qf)[HD / 16],
                                        const x8<__bf16>& baug = x8<__bf16>{}, int aug_off = 0) {
  using T = Tile<HD, 4>;  // row pitches only: the same for every wave count
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < HD / 16; ++kk) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const x8<E> a = *(const __attribute__((address_space(3))) x8<E>*)(kt + 32 * kb * T::KPITCH + 32 * kk);
      s[kb] = mfma32(a, qf[kk], s[kb]);
    }
  }
  if constexpr (AUG) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const x8<__bf16> a = *(const __attribute__((address_space(3))) x8<__bf16>*)(kt + aug_off + 32 * kb * T::KPITCH);
      s[kb] = mfma32(a, baug, s[kb]);
    }
  }
}

// A operand of O^T += V^T P^T for column block db and key chunk ci: V^T[d][16ci + 8*(lane/32) + 0..7]
// for d = 32db + lane%32.  `vt` is this lane's transpose-read address in a V buffer
// (see vt_lane_offset); each read returns 4 consecutive keys of one column.
template <int HD, typename E>
__device__ __forceinline__ x8<E> v_operand(const lds_u8* vt, int db, int ci) {
  using T = Tile<HD, 4>;  // row pitches only: the same for every wave count
  const s16x4 lo = lds_read_tr(vt + 16 * ci * T::VPITCH + T::VBLOCK * db);
  const s16x4 hi = lds_read_tr(vt + (16 * ci + 4) * T::VPITCH + T::VBLOCK * db);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(x8<E>, both);
}

// Byte offset of this lane's transpose reads in a V buffer.  Within each group of
// 16 lanes, lane 4e + q reads 4 columns of key row e: the transpose then hands lane
// j of the group keys 0..3 of column j.  Groups: lanes 0-15 columns 0-15, 16-31
// columns 16-31 (keys +0..7), 32-47 and 48-63 the same columns for keys +8..15.
template <int HD>
__device__ __forceinline__ int vt_lane_offset(int lane) {
  using T = Tile<HD, 4>;  // row pitches only: the same for every wave count
  const int g = lane >> 4, r = lane & 15;
  return (8 * (g >> 1) + (r >> 2)) * T::VPITCH + (16 * (g & 1) + 4 * (r & 3)) * 2;
}

// ALiBi (page "2.4"): the bias -slope * |pos - key| of key j0 + 8*half + koff, koff =
// 32kb + 16(r/8) + r%8, is linear in koff on a tile whose keys all lie on one side of
// the row's position: slope * koff + b to the left, with b = slope * (j0 + 8*half -
// pos), and -slope * koff - b to the right.  The scores stay in raw units with the
// koff part folded in, t = s + (+-slope / c) * koff (one FMA per score); the per-lane
// part b is carried beside the tile, so that t * c + b is the biased score in log2
// units (exact row max, and p = exp2(t * c + b - m) in one FMA as without ALiBi).  A
// tile that straddles a row's position takes the left form; its keys right of the
// position (visible only without a causal mask) then get -2 * slope * (key - pos) / c
// more, which makes their bias exact.  slope and c here are in log2 units.
template <bool DIV>
__device__ __forceinline__ void bias_tile(f32x16 (&s)[2], float slope, float c, float slope_c, int j0, int my_pos,
                                          int half, bool right, bool straddle) {
  // slope_c = slope / c, formed once per row (DIV: divided here, see prep_scores)
  const float gc = DIV ? (right ? -slope : slope) / c : (right ? -slope_c : slope_c);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(gc, (float)(32 * kb + 16 * (r >> 3) + (r & 7)), s[kb][r]);
  }
  if (straddle) {
    const float dpos = (float)(my_pos - j0 - 8 * half);  // pos - key = dpos - koff
    const float k2 = DIV ? 2.f * slope / c : 2.f * slope_c;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[kb][r] = fmaf(k2, fminf(dpos - (float)(32 * kb + 16 * (r >> 3) + (r & 7)), 0.f), s[kb][r]);
    }
  }
}

// Set the scores of keys this row may not see to -inf (tiles crossing a mask
// boundary).  The row sees the key interval [lo, hi]; element (kb, r) of this lane
// holds key j0 + 8*half + c with c = 32kb + 16(r/8) + r%8, so visibility is one
// unsigned compare of (j0 + 8*half - lo) + c against hi - lo.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int j0, int key_hi, int my_pos, int wl, int wr, int half) {
  const int lo = wl < 0 ? 0 : max(0, my_pos - wl);
  const int hi = wr < 0 ? key_hi - 1 : min(key_hi - 1, my_pos + wr);
  int d = j0 + 8 * half - lo;
  int span = hi - lo;
  if (span < 0) {  // nothing visible: every (d + c) must compare above span = 0
    span = 0;
    d = -(1 << 20);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int cidx = 32 * kb + 16 * (r >> 3) + (r & 7);
      const bool vis = (uint32_t)(d + cidx) <= (uint32_t)span;
      s[kb][r] = vis ? s[kb][r] : -INFINITY;
    }
  }
}

// Max of the scores in log2 units: the stored max times `cs` (> 0); -inf stays -inf.
__device__ __forceinline__ float to_log2(float mx, float cs) { return mx == -INFINITY ? mx : mx * cs; }

// Max of this lane's 32 scores of the tile (v_maximum3 tree; no NaN reaches here
// from finite inputs).
__device__ __forceinline__ float lane_max(const f32x16 (&s)[2]) {
  typedef float f32x32 __attribute__((ext_vector_type(32)));
  const f32x32 all = __builtin_shufflevector(s[0], s[1], 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16,
                                             17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31);
  return __builtin_reduce_maximum(all);
}

// Row max over the tile: this lane's 32 scores, then the other half-wave's 32.
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) { return max_with_other_half(lane_max(s)); }

// Instruction-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200,
              SG_TRANS = 0x400;

// Per-wave state of the forward loop.
template <int HD, typename E>
struct FwdState {
  x8<E> qf[HD / 16];       // Q^T fragments (B operand of S^T = K Q^T)
  f32x16 oacc[HD / 32];     // O^T accumulator, unscaled
  float m_run;              // reference maximum of the exponentials (log2 units)
  float l_run;              // this lane's share of the row sum against m_run
  float b_cur;              // log2 offset to add to the stored scores of the tile in s_cur (ALiBi)
  x8<__bf16> baug;          // B operand of the bias product (qk_tile, AUG)
  int aug_off;              // byte offset of this lane's pad slot from its K operand address
};

// Prepare the raw S^T of tile t (first key j0): with ALiBi fold in the bias (bias_tile)
// and set this lane's log2 offset b; mask where the tile crosses a mask boundary.
// Stored scores times `cs`, plus b, are the scores in log2 units.  Returns the tile's
// row max in log2 units.
// slope_c = slope / cs is formed once per row by the caller, except at headdim 256
// (DIV): there the one-wave-per-SIMD kernel ran 17% slower with any other form than
// with both divisions of bias_tile on every tile.
// AUG (causal ALiBi, keys right to left): the products already added slope/cs times the
// key's index in the tile, so only the offset b = slope * (j0 - position) remains; every
// visible key is at or left of the row's position, where that linear form is exact.
template <bool ALIBI, bool DIV = false, bool AUG = false>
__device__ __forceinline__ float prep_scores(f32x16 (&s)[2], float& b, int j0, int key_hi, int my_pos, int wl, int wr,
                                             int i0, int i_last, int off, float cs, float slope, float slope_c,
                                             int half) {
  const bool full =
      (j0 + BC <= key_hi) && (wl < 0 || j0 >= i_last + off - wl) && (wr < 0 || j0 + BC - 1 <= i0 + off + wr);
  b = 0.f;
  if constexpr (AUG) {
    b = slope * (float)(j0 - my_pos);
  } else if constexpr (ALIBI) {
    const bool left = j0 + BC - 1 <= i0 + off;  // every key at or before every row's position
    const bool right = j0 >= i_last + off;      // every key at or after every row's position
    const bool rgt = right && !left;
    const float d = slope * (float)(j0 + 8 * half - my_pos);
    b = rgt ? -d : d;
    // on a straddling tile the keys right of a row's position are visible only
    // without a causal mask (wr != 0)
    bias_tile<DIV>(s, slope, cs, slope_c, j0, my_pos, half, rgt, !left && !right && wr != 0);
  }
  if (!full) mask_tile(s, j0, key_hi, my_pos, wl, wr, half);
  const float mx = to_log2(lane_max(s), cs);
  // the two half-waves hold different keys, so each adds its own offset first
  return max_with_other_half(mx == -INFINITY ? mx : mx + b);
}

// Reference maximum kept without a per-tile row max (kernels without ALiBi): P(t) is
// formed against the current reference; only when the tile's exponentials grow past
// 2^16 in some lane's partial sum (or overflow), which only rising scores cause, or
// when a row whose reference is still -inf (no visible key so far; its P(t) was formed
// against 0) sees a visible key, does the tile's exact row max replace the reference, with O
// and l rescaled and P(t) formed again.  The result is unchanged: O, l and the
// logsumexp share one reference, whatever it is, and every row with a visible key ends
// with a finite one.  Returns the new partial sums through lsum0/lsum1.
template <int HD, typename E>
__device__ __forceinline__ void refit_reference(FwdState<HD, E>& st, const f32x16 (&s_cur)[2], x8<E> (&pf)[4],
                                                float cs, float& lsum0, float& lsum1) {
  bool refit = !(lsum0 + lsum1 <= 65536.f);
  // a row still without a reference: any visible (finite) score of the tile, even one
  // whose exponential against 0 underflowed, gives it one
  if (st.m_run == -INFINITY) refit = refit || lane_max(s_cur) != -INFINITY;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(refit) != 0, 0)) {
    const float mt = max_with_other_half(to_log2(lane_max(s_cur), cs) + st.b_cur);
    const float m_new = fmaxf(st.m_run, mt);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
    st.m_run = m_new;
    const float negm2 = (m_new == -INFINITY) ? 0.f : st.b_cur - m_new;
    lsum0 = 0.f;
    lsum1 = 0.f;
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) {
      const int kb = ci >> 1, r0 = 8 * (ci & 1);
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(s_cur[kb][r0 + 2 * e], cs, negm2));
        const float p1 = fast_exp2(fmaf(s_cur[kb][r0 + 2 * e + 1], cs, negm2));
        pk[e] = pack2<E>(p0, p1);
        lsum0 += p0;
        lsum1 += p1;
      }
      pf[ci] = __builtin_bit_cast(x8<E>, u32x4{pk[0], pk[1], pk[2], pk[3]});
    }
  }
}

// LDS buffers of the forward loop, as byte addresses.
struct LdsBufs {
  lds_u8* k[3];        // K tile buffers (NBUF used)
  lds_u8* v[3];        // V tile buffers
  const lds_u8* kl[3]; // this lane's K operand address in each K buffer
  const lds_u8* vl[3]; // this lane's transpose-read address in each V buffer
};

// One tile step: P(t) from s_cur, S(t+1) into s_nxt, O += V(t) P(t), loads of
// K(t+2) and V(t+1) into the free buffers, reference-maximum update.  Ends with
// the tile barrier.  The last step of an item (LAST) only forms P(t) and adds
// V(t) P(t): there is no next tile to score or load, and no buffer to hand over.
template <int HD, int NW, bool ALIBI, typename E, bool LAST, int PAR, typename KV>
__device__ __forceinline__ void tile_step(FwdState<HD, E>& st, const f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], int t,
                                          int t_begin, const KV& kv, const LdsBufs& lb, int half,
                                          float slope_c, float cs, float slope, int my_pos, int wl, int wr, int i0,
                                          int i_last, int off) {
  using T = Tile<HD, NW>;
  constexpr int NB = T::NBUF;
  // Tile j lives in buffer (j - t_begin) % NB.  This step reads K(t+1) and V(t) and
  // loads K(t+NB) and V(t+NB-1) into the buffers K(t) and V(t-1) left (both read in
  // the previous step).  Past the last tile these loads read zeros or unused keys.
  // (with two buffers the step's parity PAR, t - t_begin mod 2, picks them at compile time)
  const int rel = t - t_begin;
  const int b0 = NB == 2 ? PAR : rel % NB, b1 = NB == 2 ? 1 - PAR : (rel + 1) % NB,
            bm1 = NB == 2 ? 1 - PAR : (rel + NB - 1) % NB;
  if constexpr (!LAST) {
    kv.load_k(lb.k[b0], t + NB);
    kv.load_v(lb.v[bm1], t + NB - 1);
  }
  if constexpr (std::is_same_v<KV, PagedKVStream<HD, NW>>) {
    // decode form: a wave none of whose rows exists only streams tiles for the others
    // (and meets the others at the tile barrier, which the last step does not have)
    if (!kv.active) {
      if constexpr (!LAST) {
        wait_tile_loads<NB == 2 ? 0 : T::MIN_LOADS_PER_STEP>();
        __syncthreads();
      }
      return;
    }
  }

  // S(t+1) = K(t+1) Q^T
  constexpr bool AUG = ALIBI && KV::KEEP_PAD;
  if constexpr (!LAST) qk_tile<HD, E, AUG>(s_nxt, lb.kl[b1], st.qf, st.baug, st.aug_off);

  // P(t) = exp2(S(t) * cs - m), rounded to E for the P V product
  const float negm = (st.m_run == -INFINITY) ? 0.f : st.b_cur - st.m_run;
  x8<E> pf[4];
  float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
    const int kb = ci >> 1, r0 = 8 * (ci & 1);
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(fmaf(s_cur[kb][r0 + 2 * e], cs, negm));
      const float p1 = fast_exp2(fmaf(s_cur[kb][r0 + 2 * e + 1], cs, negm));
      pk[e] = pack2<E>(p0, p1);
      // the row sum stays in fp32: the lse needs it to ~1e-4 relative, which a sum
      // of bf16-rounded terms (2^-9 each) cannot guarantee
      lsum0 += p0;
      lsum1 += p1;
    }
    pf[ci] = __builtin_bit_cast(x8<E>, u32x4{pk[0], pk[1], pk[2], pk[3]});
  }
  // (not at headdim 256: there the one-wave-per-SIMD kernel with its accumulators in
  // the AGPRs ran 23% slower with the refit code in the loop)
  constexpr bool NOMAX = !ALIBI && FA_NOMAX && HD != 256;
  if constexpr (NOMAX) refit_reference<HD, E>(st, s_cur, pf, cs, lsum0, lsum1);
  // At headdim 256 (one wave per SIMD) keep the row-sum adds in this block, between
  // the products; left alone they sink past the masking branch below.  With two
  // waves per SIMD the sunk adds overlap the other wave's products, which measured
  // faster at headdim 64 and 128.
  if constexpr (HD == 256) asm volatile("" : "+v"(lsum0), "+v"(lsum1));
  st.l_run += lsum0 + lsum1;

  // O^T += V(t)^T P(t)^T
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) {
      const x8<E> a = v_operand<HD, E>(lb.vl[b0], db, ci);
      st.oacc[db] = mfma32(a, pf[ci], st.oacc[db]);
    }
  }

  if constexpr (LAST) {
    // each product's two operand reads issued one product ahead
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
#pragma unroll
    for (int i = 0; i + 1 < HD / 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    return;
  }

  // max of S(t+1) before masking: exact for tiles every row sees in full
  const int j1 = kv.tile_key(t + 1);
  float mx = 0.f;  // row max of S(t+1) in log2 units
  if constexpr (!ALIBI && !NOMAX) mx = to_log2(tile_max(s_nxt), cs);

  // Issue order: the global loads; LDS operand reads running four products ahead;
  // the S(t+1) products, each followed by two exponentials of tile t and their
  // FMAs/conversions; then the P V products, each followed by row-sum adds, the
  // max of S(t+1), the V transposition and the LDS stores.
  constexpr int NQK = HD / 8;  // products per phase (S(t+1), then P V)
#ifndef FA_SCHED
#define FA_SCHED 1
#endif
  if constexpr (FA_SCHED == 2) {
    __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, T::LOADS_PER_STEP, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 4, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_TRANS, 32 / NQK, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
    }
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, 5, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
    }
  } else if constexpr (FA_SCHED == 1) {
#ifndef FA_V1_256
#define FA_V1_256 4
#endif
#ifndef FA_V2_256
#define FA_V2_256 5
#endif
#ifndef FA_PF_256
#define FA_PF_256 12
#endif
    // vector instructions placed after each product of the S(t+1) phase (V1) and of the
    // P V phase (V2); headdim 256 (one wave per SIMD, 32 products per phase) measured
    // +11% with four instead of three after each S product, which leaves room for all of
    // tile t's exponentials inside the first phase
    constexpr int FA_V1 = HD == 256 ? FA_V1_256 : 3;  // headdim 64: 3-14 all within 1%
    constexpr int FA_V2 = HD == 256 ? FA_V2_256 : 5;
    // LDS operand reads issued ahead of the first product: at headdim 256 only one
    // wave runs per SIMD, so a deeper queue hides more LDS latency.
    constexpr int FA_PF = HD == 256 ? FA_PF_256 : 2;
#ifndef FA_VI
#define FA_VI 0
#endif
    __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, T::LOADS_PER_STEP, 0);
    if constexpr (FA_PF > 0) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, FA_PF, 0);
    // exponentials of tile t fill the first LDS latency after the barrier
    if constexpr (FA_VI > 0) __builtin_amdgcn_sched_group_barrier(SG_VALU, FA_VI, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, FA_V1, 0);
    }
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, FA_V2, 0);
    }
  }

  // ALiBi tiles, and tiles crossing a mask boundary: bias / mask, then take the max again
  float b_nxt = 0.f;
  if constexpr (ALIBI) {
    mx = prep_scores<ALIBI, HD == 256, AUG>(s_nxt, b_nxt, j1, kv.key_hi, my_pos, wl, wr,
                                            i0, i_last, off, cs, slope, slope_c, half);
  } else {
    const bool nxt_full = (j1 + BC <= kv.key_hi) && (wl < 0 || j1 >= i_last + off - wl) &&
                          (wr < 0 || j1 + BC - 1 <= i0 + off + wr);
    if (!nxt_full)
      mx = prep_scores<ALIBI, HD == 256>(s_nxt, b_nxt, j1, kv.key_hi, my_pos, wl, wr,
                                         i0, i_last, off, cs, slope, slope_c, half);
  }
  st.b_cur = b_nxt;  // tile t's offset was used by P(t) above

  // move the reference maximum only when a row grew by more than 2^8 (without ALiBi,
  // refit_reference moves it instead, on the next step's exponentials)
  const float m_new = fmaxf(st.m_run, mx);
  if (!NOMAX && __builtin_expect(__builtin_amdgcn_ballot_w64(m_new > st.m_run + RESCALE_TH) != 0, 0)) {
    // 0 when only m_run is -inf; 1 for a row that has seen no visible key yet
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
    st.m_run = m_new;
  }
  // K(t+2) and V(t+1) (loaded NB-2 steps ago) are in LDS before anyone passes the barrier
  wait_tile_loads<NB == 2 ? 0 : T::MIN_LOADS_PER_STEP>();
  __syncthreads();
}

// ---- ping-pong schedule of the eight-wave workgroup ---------------------------------
// The four-wave step above has every wave do the same thing at the same time: all
// waves form S(t+1) and the exponentials of P(t) (matrix products and vector work,
// K operand reads), then all waves form O += V(t) P(t) (matrix products and V
// transpose reads), with one barrier per step.  The V transpose reads of all eight
// waves then fall into the same half of the step, where LDS bounds it.  Here waves
// 0-3 (group A, the K loaders) run half a step ahead of waves 4-7 (group B, the V
// loaders), with a barrier every half step: while one group is in its first half the
// other is in its second, so every SIMD (one wave of each group) always has one wave
// issuing exponentials and one issuing V reads beside the matrix products.
//
// Half-step h: group A runs half 1 of step h/2 (even h) or half 2 (odd h); group B the
// same one half-step later.  Buffers (two per tensor, tile j in buffer (j - t_begin) % 2):
//  * K(t+2) is loaded by group A in its half 1 of step t (h = 2t) into K(t)'s buffer,
//    whose last reader was group B's half 1 of step t-1 (h = 2t-1); group A waits for
//    it in its half 2 (h = 2t+1); the first reader is group A at h = 2t+2;
//  * V(t+1) is loaded by group B in its half 1 of step t (h = 2t+1) into V(t-1)'s
//    buffer, last read by group B's half 2 of step t-1 (h = 2t); group B waits for it
//    in its half 2 (h = 2t+2); the first reader is group A at h = 2t+3.
// The half-step barrier is a plain s_barrier: no fence, so it does not wait for the
// tile loads still in flight (each loading wave waits for its own before the barrier
// that precedes their first reader).  Its memory clobber keeps the compiler from
// moving LDS accesses across it, and the scheduling barriers keep every other
// instruction (the matrix products included) on its own side.
__device__ __forceinline__ void half_step_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Half 1 of step t: loads, S(t+1) = K(t+1) Q^T, P(t) (rounded to E into pf) and its row sum.
template <int HD, typename E, bool LAST, int PAR, bool NOMAX>
__device__ __forceinline__ void pp_half1(FwdState<HD, E>& st, const f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                                         x8<E> (&pf)[4], int t, const KVStream<HD, 8>& kv, const LdsBufs& lb,
                                         float cs) {
  using T = Tile<HD, 8>;
  if constexpr (!LAST) {
    kv.load_k(lb.k[PAR], t + 2);      // group A only
    kv.load_v(lb.v[1 - PAR], t + 1);  // group B only
    qk_tile<HD, E>(s_nxt, lb.kl[1 - PAR], st.qf);
  }
  const float negm = (st.m_run == -INFINITY) ? 0.f : st.b_cur - st.m_run;
  float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
    const int kb = ci >> 1, r0 = 8 * (ci & 1);
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(fmaf(s_cur[kb][r0 + 2 * e], cs, negm));
      const float p1 = fast_exp2(fmaf(s_cur[kb][r0 + 2 * e + 1], cs, negm));
      pk[e] = pack2<E>(p0, p1);
      lsum0 += p0;
      lsum1 += p1;
    }
    pf[ci] = __builtin_bit_cast(x8<E>, u32x4{pk[0], pk[1], pk[2], pk[3]});
  }
  if constexpr (NOMAX) refit_reference<HD, E>(st, s_cur, pf, cs, lsum0, lsum1);
  st.l_run += lsum0 + lsum1;
  if constexpr (!LAST) {
#ifndef FA_PP_V1
#define FA_PP_V1 7
#endif
#ifndef FA_PP_PF1
#define FA_PP_PF1 2
#endif
    // the loads; K operand reads FA_PP_PF1 products ahead; each S product followed by
    // FA_PP_V1 vector instructions of P(t) (112 of them: FMA, exponential, row-sum add
    // per score and one conversion per pair)
    __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, T::LOADS_PER_STEP, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, FA_PP_PF1, 0);
#pragma unroll
    for (int i = 0; i < HD / 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_VALU, FA_PP_V1, 0);
    }
  }
}

// Half 2 of step t: O += V(t) P(t); then (unless LAST) the max of S(t+1) with its mask
// and bias, the reference-maximum update, and the wait for this wave's tile loads.
template <int HD, bool ALIBI, typename E, bool LAST, int PAR>
__device__ __forceinline__ void pp_half2(FwdState<HD, E>& st, f32x16 (&s_nxt)[2], const x8<E> (&pf)[4], int t,
                                         const KVStream<HD, 8>& kv, const LdsBufs& lb, int half, float slope_c,
                                         float cs, float slope, int my_pos, int wl, int wr, int i0, int i_last,
                                         int off) {
#pragma unroll
  for (int ci = 0; ci < 4; ++ci) {
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) {
      const x8<E> a = v_operand<HD, E>(lb.vl[PAR], db, ci);
      st.oacc[db] = mfma32(a, pf[ci], st.oacc[db]);
    }
  }
#ifndef FA_PP_V2
#define FA_PP_V2 2
#endif
#ifndef FA_PP_PF2
#define FA_PP_PF2 4
#endif
  // V transpose reads FA_PP_PF2 ahead (two per product), FA_PP_V2 vector instructions
  // (the row max of S(t+1)) after each product
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, FA_PP_PF2, 0);
#pragma unroll
  for (int i = 0; i < HD / 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_VALU, FA_PP_V2, 0);
  }
  if constexpr (LAST) return;

  const int j1 = kv.tile_key(t + 1);
  float mx = 0.f;
  float b_nxt = 0.f;
  if constexpr (!ALIBI && FA_NOMAX) {
    // the mask only; the reference maximum moves in half 1 when needed (refit_reference)
    const bool nxt_full = (j1 + BC <= kv.key_hi) && (wl < 0 || j1 >= i_last + off - wl) &&
                          (wr < 0 || j1 + BC - 1 <= i0 + off + wr);
    if (!nxt_full)
      (void)prep_scores<ALIBI, HD == 256>(s_nxt, b_nxt, j1, kv.key_hi, my_pos, wl, wr,
                                          i0, i_last, off, cs, slope, slope_c, half);
    st.b_cur = b_nxt;
    wait_tile_loads<0>();
    return;
  }
  if constexpr (ALIBI) {
    mx = prep_scores<ALIBI, HD == 256>(s_nxt, b_nxt, j1, kv.key_hi, my_pos, wl, wr,
                                       i0, i_last, off, cs, slope, slope_c, half);
  } else {
    mx = to_log2(tile_max(s_nxt), cs);
    const bool nxt_full = (j1 + BC <= kv.key_hi) && (wl < 0 || j1 >= i_last + off - wl) &&
                          (wr < 0 || j1 + BC - 1 <= i0 + off + wr);
    if (!nxt_full)
      mx = prep_scores<ALIBI, HD == 256>(s_nxt, b_nxt, j1, kv.key_hi, my_pos, wl, wr,
                                         i0, i_last, off, cs, slope, slope_c, half);
  }
  st.b_cur = b_nxt;
  const float m_new = fmaxf(st.m_run, mx);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(m_new > st.m_run + RESCALE_TH) != 0, 0)) {
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
    st.m_run = m_new;
  }
  // the tile loads this wave issued in its half 1 have landed before the next barrier
  wait_tile_loads<0>();
}

// One step in the ping-pong order: half 1, barrier, half 2, barrier.
template <int HD, bool ALIBI, typename E, bool LAST, int PAR>
__device__ __forceinline__ void pp_step(FwdState<HD, E>& st, const f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                                        x8<E> (&pf)[4], int t, const KVStream<HD, 8>& kv, const LdsBufs& lb,
                                        int half, float slope_c, float cs, float slope, int my_pos, int wl, int wr,
                                        int i0,
                                        int i_last, int off) {
  pp_half1<HD, E, LAST, PAR, !ALIBI && FA_NOMAX>(st, s_cur, s_nxt, pf, t, kv, lb, cs);
  half_step_barrier();
  pp_half2<HD, ALIBI, E, LAST, PAR>(st, s_nxt, pf, t, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr, i0, i_last,
                                    off);
  half_step_barrier();
}

// One work item: (batch, head, query tile[, key split]) number `item` of `items`.
// DEC (KV-cache decode, split mode only): the block's rows are the Sq * G queries that
// share K/V head h (G = nheads / nheads_k query heads, row r = query i * G + head g),
// read from a KV cache (Sk = cache_seqlens[b] + seqlen_new keys, paged through the block
// table or contiguous); every K/V tile loaded then serves all of them.
// REV: key tiles right to left (the ALiBi kernels under a causal mask, see launch_fwd_hd).
template <int HD, int NW, bool ALIBI, bool SPLIT, typename E, bool DEC = false, bool REV = false>
__device__ __forceinline__ void fwd_item(const FwdParams& p, uint8_t* smem, int item, int items) {
  static_assert(!DEC || SPLIT, "the decode form writes split partials");
  using T = Tile<HD, NW>;
  constexpr int BR = 32 * NW;  // query rows per workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lrow = lane & 31;  // query column / A-operand row owned by this lane
  const int half = lane >> 5;  // which 8-element k slice this lane feeds

  // ---- work item -------------------------------------------------------------
  // Items run query tile fastest, then key split, batch, and head slowest.  Each XCD
  // takes a contiguous range of items (xcd_remap), i.e. a slice of the heads over
  // every sequence of the batch: the XCDs then get equal work even when sequences
  // differ in length, and the query heads that share a K/V head stay on one XCD.
  // Padded batches with a causal mask or right window (tiles of unequal length)
  // take the heavy-first order of heavy_first_item instead: groups of up to four
  // (batch, head) pairs, query tile slowest and heaviest first inside a group, so
  // no heavy tile of the last heads starts late.
  int qt, split = 0, b, h;
  if (!SPLIT && p.reverse_q && p.cu_q == nullptr) {
    const int bh = heavy_first_item(xcd_remap(item, items), p.num_q_tiles, p.batch * p.nheads, qt);
    qt = p.num_q_tiles - 1 - qt;
    b = bh % p.batch;
    h = bh / p.batch;
  } else {
    int w = xcd_remap(item, items);
    qt = w % p.num_q_tiles;
    w /= p.num_q_tiles;
    if constexpr (SPLIT) {
      split = w % p.num_splits;
      w /= p.num_splits;
    }
    b = w % p.batch;
    h = w / p.batch;
    if (p.reverse_q) qt = p.num_q_tiles - 1 - qt;
  }

  // This sequence's rows: a padded batch has them at b * seqlen; a packed (varlen)
  // batch lists each sequence's first row in cu_q / cu_k.
  long q_start, k_start;
  int Sq, Sk;
  if (DEC) {
    Sq = p.seqlen_q;
    Sk = p.cache_seqlens[b] + p.seqlen_new;
    q_start = (long)b * Sq;
    k_start = p.block_table != nullptr ? 0 : (long)b * p.page_size;  // contiguous: page_size = capacity
  } else if (p.cu_q != nullptr) {
    q_start = p.cu_q[b];
    Sq = p.cu_q[b + 1] - q_start;
    k_start = p.cu_k[b];
    Sk = p.cu_k[b + 1] - k_start;
    if (qt * BR >= Sq) return;  // the whole workgroup: no row of this tile exists
  } else {
    Sq = p.seqlen_q;
    Sk = p.seqlen_k;
    q_start = (long)b * Sq;
    k_start = (long)b * Sk;
  }
  int key_lo = 0, key_hi = Sk;
  if constexpr (SPLIT) {
    key_lo = min(Sk, split * p.split_len);
    key_hi = min(Sk, key_lo + p.split_len);
  }
  const long row_stride = (long)p.nheads * HD;     // q and out
  const long kv_stride = (long)p.nheads_k * HD;    // k and v
  const int G = p.nheads / p.nheads_k;
  const int hk = DEC ? h : h / G;                  // the decode form's items are K/V heads
  const uint16_t* __restrict__ qbase = p.q + q_start * row_stride + (long)h * HD;

  std::conditional_t<DEC, PagedKVStream<HD, NW>, KVStream<HD, NW, REV>> kv;
  kv.kbase = p.k + k_start * kv_stride + (long)hk * HD;
  kv.vbase = p.v + k_start * kv_stride + (long)hk * HD;
  kv.key_lo = key_lo;
  kv.key_hi = key_hi;
  kv.row_stride = (int)kv_stride;
  kv.row_bytes = (int)kv_stride * 2;
  if constexpr (DEC) {
    kv.btab = p.block_table != nullptr ? p.block_table + (long)b * p.max_blocks : nullptr;
    kv.page_shift = p.page_shift;
    kv.active = qt * BR + wave * 32 < Sq * G;
  }
  kv.init(wave, lane);

  LdsBufs lb;
  lds_u8* const lds = (lds_u8*)smem;
#pragma unroll
  for (int i = 0; i < T::NBUF; ++i) {
    lb.k[i] = lds + i * T::KBYTES;
    lb.v[i] = lds + T::NBUF * T::KBYTES + i * T::VBYTES;
    lb.kl[i] = lb.k[i] + lrow * T::KPITCH + 16 * half;
    lb.vl[i] = lb.v[i] + vt_lane_offset<HD>(lane);
  }

  // Positions (query index i) of the block's first and last row; the decode form's
  // rows r = i * G + g of rows_total = Sq * G hold G heads per position.
  const int rows_total = DEC ? Sq * G : Sq;
  const int r0 = qt * BR;
  const int i0 = DEC ? r0 / G : r0;
  const int i_last = DEC ? (min(r0 + BR, rows_total) - 1) / G : min(r0 + BR, Sq) - 1;
  const int off = Sk - Sq;  // query i sits at key position i + off
  const int wl = p.window_left, wr = p.window_right;
  // Positions of this wave's first and last row: the per-tile mask and ALiBi tests use
  // them, so a tile that crosses a mask boundary only within the other waves' rows is a
  // full tile for this wave (a wave of 32 rows meets about half as many boundary tiles
  // as the block of 128).  A wave whose rows are all past the end takes the last row.
#ifndef FA_WAVE_TESTS
#define FA_WAVE_TESTS 1
#endif
  const int wr0 = r0 + wave * 32;
  const int i0w = FA_WAVE_TESTS ? (DEC ? min(wr0, rows_total - 1) / G : min(wr0, Sq - 1)) : i0;
  const int ilw = FA_WAVE_TESTS ? (DEC ? min(wr0 + 31, rows_total - 1) / G : min(wr0 + 31, Sq - 1)) : i_last;

  // Key tiles that any row of this block can see.
  int lo = key_lo, hi = key_hi - 1;
  if (wl >= 0) lo = max(lo, i0 + off - wl);
  if (wr >= 0) hi = min(hi, i_last + off + wr);
  int t_begin = 0, t_end = 0;
  if (hi >= lo) {
    t_begin = (lo - key_lo) / BC;
    t_end = (hi - key_lo) / BC + 1;
  }
  kv.t_sum = t_begin + t_end - 1;
  kv.t_stop = t_end;

  // ---- Q fragments: B operand of S^T = K Q^T, held for the whole loop ----------
  FwdState<HD, E> st;
  const int my_r = r0 + wave * 32 + lrow;         // this lane's row of the block
  const int my_q = DEC ? my_r / G : my_r;         // its query index
  const int my_h = DEC ? hk * G + my_r % G : h;   // and its query head
  const bool my_valid = my_r < rows_total;
  const int my_pos = my_q + off;
  const uint16_t* __restrict__ my_qrow =
      DEC ? p.q + (((long)b * Sq + my_q) * p.nheads + my_h) * HD : qbase + (long)my_q * row_stride;
#pragma unroll
  for (int kk = 0; kk < HD / 16; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_valid) raw = *(const u32x4*)(my_qrow + 16 * kk + 8 * half);
    raw = (raw & p.q_and) ^ p.q_sign;
    st.qf[kk] = __builtin_bit_cast(x8<E>, raw);
  }
#pragma unroll
  for (int db = 0; db < HD / 32; ++db) st.oacc[db] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.b_cur = 0.f;
  const float c = p.scale_log2;
  float slope = 0.f;
  if constexpr (ALIBI) slope = p.alibi[(long)b * p.alibi_bstride + my_h] * kLog2e;  // bias in log2 units
  // the bias step per key in raw score units (bias_tile); headdim 256 divides per tile
  const float slope_c = (ALIBI && HD != 256) ? slope / c : 0.f;
  // multiplier turning the stored scores into log2 units
  const float cs = c;
  constexpr bool AUG = ALIBI && decltype(kv)::KEEP_PAD;
  if constexpr (AUG) {
    // the bias step per key in raw score units, g = slope / c, as three bf16 parts
    // (their sum is g to about 24 bits): the B operand of the bias product
    const float g = slope / c;
    const float g_hi = widen_lo<__bf16>(pack2<__bf16>(g, 0.f));
    const float g_mid = widen_lo<__bf16>(pack2<__bf16>(g - g_hi, 0.f));
    const float g_lo = g - g_hi - g_mid;
    const u32x4 bq = half == 0 ? u32x4{pack2<__bf16>(g_hi, g_mid), pack2<__bf16>(g_lo, 0.f), 0u, 0u}
                               : u32x4{0u, 0u, 0u, 0u};
    st.baug = __builtin_bit_cast(x8<__bf16>, bq);
    st.aug_off = 2 * HD - 16 * half;
    // A operand: the pad slot of LDS row r holds its key index k_lds_row(r) three times
    // (exact in bf16), then zeros; written once per K buffer, the loads skip those slots
    if (tid < T::NBUF * BC) {
      const int r = tid % BC;
      const float k = (float)k_lds_row(r);
      *(__attribute__((address_space(3))) u32x4*)(lds + (tid / BC) * T::KBYTES + r * T::KPITCH + 2 * HD) =
          u32x4{pack2<__bf16>(k, k), pack2<__bf16>(k, 0.f), 0u, 0u};
    }
  }

  f32x16 s_a[2], s_b[2];

  if (t_begin < t_end) {
    // prologue: K of the first NBUF tiles and V of the first NBUF-1, then S of the
    // first (tiles past the last key land as zeros: harmless)
#pragma unroll
    for (int j = 0; j < T::NBUF; ++j) kv.load_k(lb.k[j], t_begin + j);
#pragma unroll
    for (int j = 0; j + 1 < T::NBUF; ++j) kv.load_v(lb.v[j], t_begin + j);
    wait_tile_loads<0>();
    __syncthreads();
    qk_tile<HD, E, AUG>(s_a, lb.kl[0], st.qf, st.baug, st.aug_off);
    const int j0 = kv.tile_key(t_begin);
    st.m_run = prep_scores<ALIBI, HD == 256, AUG>(s_a, st.b_cur, j0, key_hi, my_pos, wl, wr,
                                             i0w, ilw, off, cs, slope, slope_c, half);
    __syncthreads();  // every wave is done with K(t_begin) before the loop refills its buffer
  }

  // two tiles per trip so S(t) and S(t+1) swap roles without register copies.  Where
  // the registers allow it (headdim 128, and 64 except the split ALiBi form, outside
  // the decode form) the item's last tile takes the short LAST step: +1-3.5% on 2k-4k
  // launches; elsewhere its extra code spilled in the loop.
  constexpr bool SHORT_LAST = !DEC && (HD == 128 || (HD == 64 && (!ALIBI || !SPLIT)));
#ifndef FA_PINGPONG
#define FA_PINGPONG 1
#endif
  if constexpr (NW == 8 && FA_PINGPONG && !DEC && !SPLIT) {
    // eight waves: the ping-pong order (group B starts half a step behind group A and
    // ends half a step after it; both pass the same number of barriers)
    const bool group_a = wave < 4;
    x8<E> pf[4];
    if (!group_a) half_step_barrier();
    int t = t_begin;
    for (; t + 2 < t_end; t += 2) {
      pp_step<HD, ALIBI, E, false, 0>(st, s_a, s_b, pf, t, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr, i0w, ilw,
                                      off);
      pp_step<HD, ALIBI, E, false, 1>(st, s_b, s_a, pf, t + 1, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr, i0w,
                                      ilw, off);
    }
    if (t + 1 < t_end) {
      pp_step<HD, ALIBI, E, false, 0>(st, s_a, s_b, pf, t, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr, i0w, ilw,
                                      off);
      pp_step<HD, ALIBI, E, true, 1>(st, s_b, s_a, pf, t + 1, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr, i0w,
                                     ilw, off);
    } else if (t < t_end) {
      pp_step<HD, ALIBI, E, true, 0>(st, s_a, s_b, pf, t, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr, i0w, ilw,
                                     off);
    }
    if (group_a) half_step_barrier();
  } else if constexpr (SHORT_LAST) {
    int t = t_begin;
    for (; t + 2 < t_end; t += 2) {
      tile_step<HD, NW, ALIBI, E, false, 0>(st, s_a, s_b, t, t_begin, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr,
                                            i0w, ilw, off);
      tile_step<HD, NW, ALIBI, E, false, 1>(st, s_b, s_a, t + 1, t_begin, kv, lb, half, slope_c, cs, slope, my_pos, wl,
                                            wr, i0w, ilw, off);
    }
    // The last step has no loads and no barrier: a wave that sees no key of the last tile
    // (a window's first rows, the rows left of a causal diagonal) skips it.
    auto wave_sees = [&](int tt) {
      const int j0 = kv.tile_key(tt);
      int klo = key_lo, khi = key_hi - 1;
      if (wl >= 0) klo = max(klo, i0w + off - wl);
      if (wr >= 0) khi = min(khi, ilw + off + wr);
      return !FA_WAVE_TESTS || (j0 <= khi && j0 + BC - 1 >= klo);
    };
    if (t + 1 < t_end) {  // two tiles left
      tile_step<HD, NW, ALIBI, E, false, 0>(st, s_a, s_b, t, t_begin, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr,
                                            i0w, ilw, off);
      if (wave_sees(t + 1))
        tile_step<HD, NW, ALIBI, E, true, 1>(st, s_b, s_a, t + 1, t_begin, kv, lb, half, slope_c, cs, slope, my_pos,
                                             wl, wr, i0w, ilw, off);
    } else if (t < t_end) {  // one tile left
      if (wave_sees(t))
        tile_step<HD, NW, ALIBI, E, true, 0>(st, s_a, s_b, t, t_begin, kv, lb, half, slope_c, cs, slope, my_pos, wl,
                                             wr, i0w, ilw, off);
    }
  } else {
    for (int t = t_begin; t < t_end; t += 2) {
      tile_step<HD, NW, ALIBI, E, false, 0>(st, s_a, s_b, t, t_begin, kv, lb, half, slope_c, cs, slope, my_pos, wl, wr,
                                            i0w, ilw, off);
      if (t + 1 >= t_end) break;
      tile_step<HD, NW, ALIBI, E, false, 1>(st, s_b, s_a, t + 1, t_begin, kv, lb, half, slope_c, cs, slope, my_pos, wl,
                                            wr, i0w, ilw, off);
    }
  }
  f32x16* const oacc = st.oacc;
  const float m_run = st.m_run;
  const float l_run = st.l_run;

  // ---- epilogue: one division per row, logsumexp ------------------------------
  const float l_tot = sum_with_other_half(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
  if (!my_valid) return;  // this lane's row is past the end: nothing to write

  if constexpr (!SPLIT) {
    uint16_t* obase = (uint16_t*)p.out + (q_start + my_q) * row_stride + (long)h * HD;
    // Accumulator rows 4g..4g+3 of block db hold columns 32db + 8g + 4*half + 0..3 of
    // this lane's row: the two half-waves hold the two 4-column halves of every 8
    // columns.  One v_permlane32_swap per packed pair hands half 0 columns 8g..8g+7
    // and half 1 columns 8g+8..8g+15, so every lane stores 16 bytes: eight stores per
    // lane at headdim 128 instead of sixteen of 8 bytes (+1.5% on 2k launches, whose
    // epilogue stores cost 3-5% of the launch; non-temporal stores were 12-23% slower).
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; g += 2) {
        const uint32_t a0 = pack2<E>(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        const uint32_t a1 = pack2<E>(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        const uint32_t b0 = pack2<E>(oacc[db][4 * g + 4] * inv, oacc[db][4 * g + 5] * inv);
        const uint32_t b1 = pack2<E>(oacc[db][4 * g + 6] * inv, oacc[db][4 * g + 7] * inv);
        // lanes 32-63 of the first operand trade with lanes 0-31 of the second
        const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
        const u32x4 o = {s0[0], s1[0], s0[1], s1[1]};
        *(u32x4*)(obase + 32 * db + 8 * (g + half)) = o;
      }
    if (half == 0) {
      const long li = p.cu_q != nullptr ? (long)h * p.lse_head_stride + q_start + my_q
                                        : ((long)b * p.nheads + h) * Sq + my_q;
      p.lse[li] = lse_v;
    }
  } else {
    const long rowid = (((long)split * p.batch + b) * p.nheads + my_h) * Sq + my_q;
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

// One workgroup per work item.  (A grid of only the resident workgroups looping
// over items with a static stride was measured slower: the causal items' unequal
// lengths then leave CUs idle.)
// Headdim 64 asks for three waves per SIMD: the register allocator then fits the ALiBi
// kernel's short last step into 168 registers (12 bytes per lane spilled) instead of
// giving up the third wave.
template <int HD, int NW, bool ALIBI, bool SPLIT, typename E, bool REV = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(HD == 64 ? 3 : 1))) void fwd_kernel(
    FwdParams p, int items) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Tile<HD, NW>::LDS_BYTES];
  fwd_item<HD, NW, ALIBI, SPLIT, E, false, REV>(p, smem, blockIdx.x, items);
}

// KV-cache decode with grouped K/V heads on the matrix cores: one workgroup per (batch,
// K/V head, key split, block of 128 rows of the Sq * G queries that share the K/V head),
// split partials as fa_fwd_splitkv writes them.
template <int HD, bool ALIBI, typename E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fwd_decode_kernel(FwdParams p,
                                                                                                int items) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Tile<HD, 4>::LDS_BYTES];
  fwd_item<HD, 4, ALIBI, true, E, true>(p, smem, blockIdx.x, items);
}

template <int HD, int NW, bool ALIBI, bool SPLIT, bool REV = false>
hipError_t launch_fwd_instance(const FwdParams& p, long nblocks, hipStream_t stream) {
  if (p.f16)
    hipLaunchKernelGGL((fwd_kernel<HD, NW, ALIBI, SPLIT, _Float16, REV>), dim3((unsigned)nblocks), dim3(64 * NW), 0,
                       stream, p, (int)nblocks);
  else
    hipLaunchKernelGGL((fwd_kernel<HD, NW, ALIBI, SPLIT, __bf16, REV>), dim3((unsigned)nblocks), dim3(64 * NW), 0,
                       stream, p, (int)nblocks);
  return hipGetLastError();
}


// One translation unit per head dimension instantiates these (separate files let
// each get its own register-allocation flags).  The caller sets num_q_tiles for
// 128-row tiles; an eight-wave launch recounts them for 256 rows.
template <int HD>
hipError_t launch_fwd_hd(const FwdParams& p, bool split, hipStream_t stream) {
  const bool alibi = p.alibi != nullptr;
  if constexpr (HD == 128) {
    if (fwd_waves(HD, split, p.window_left, p.window_right, p.seqlen_q, alibi) == 8) {
      FwdParams p8 = p;
      p8.num_q_tiles = (p.seqlen_q + 255) / 256;
      const long nblocks = (long)p8.batch * p8.nheads * p8.num_q_tiles;
      return alibi ? launch_fwd_instance<HD, 8, true, false>(p8, nblocks, stream)
                   : launch_fwd_instance<HD, 8, false, false>(p8, nblocks, stream);
    }
  }
  const long nblocks = (long)p.batch * p.nheads * p.num_q_tiles * (split ? p.num_splits : 1);
  if (split) return alibi ? launch_fwd_instance<HD, 4, true, true>(p, nblocks, stream)
                          : launch_fwd_instance<HD, 4, false, true>(p, nblocks, stream);
  // ALiBi under a causal mask (any left window): the bias only falls with distance to
  // the left of each row, so with the key tiles right to left a row's maximum is
  // reached on its first tiles and the rescaling of O that a rising maximum costs
  // (on nearly every tile of the steeper heads left to right) all but disappears:
  // +6-9% at headdim 64-256 (4k-8k rows, with and without a left window)
#ifndef FA_ALIBI_REV
#define FA_ALIBI_REV 1
#endif
  if constexpr (FA_ALIBI_REV)
    if (alibi && p.window_right == 0) return launch_fwd_instance<HD, 4, true, false, true>(p, nblocks, stream);
  return alibi ? launch_fwd_instance<HD, 4, true, false>(p, nblocks, stream)
               : launch_fwd_instance<HD, 4, false, false>(p, nblocks, stream);
}

hipError_t launch_fwd_d64(const FwdParams& p, bool split, hipStream_t stream);
hipError_t launch_fwd_d128(const FwdParams& p, bool split, hipStream_t stream);
hipError_t launch_fwd_d256(const FwdParams& p, bool split, hipStream_t stream);

// The matrix-core decode form (fwd_decode_kernel) for a KV-cache step whose K/V heads
// each serve nq_total = (nheads / nheads_k) * seqlen_q > 4 queries, headdim 64 or 128
// (decode_uses_mfma).  Up to four queries the vector-ALU kernel streams the cache
// faster (paged 32k-key caches, batch 8: 5.45 against 4.65 TB/s at four queries per
// K/V head); from eight on it falls behind (3.0 against 4.8 TB/s at eight, 1.5 against
// 3.6 at sixteen).  The caller passes split_len as a multiple of BC (so a tile never
// crosses a cache block) and the split partials as out / lse.

template <int HD>
hipError_t launch_fwd_decode_hd(const FwdParams& p, hipStream_t stream) {
  FwdParams d = p;
  d.reverse_q = 0;
  d.num_q_tiles = ((p.nheads / p.nheads_k) * p.seqlen_q + 127) / 128;
  const long nblocks = (long)d.batch * d.nheads_k * d.num_splits * d.num_q_tiles;
  const dim3 grid((unsigned)nblocks);
  if (p.f16) {
    if (p.alibi) hipLaunchKernelGGL((fwd_decode_kernel<HD, true, _Float16>), grid, dim3(256), 0, stream, d, (int)nblocks);
    else hipLaunchKernelGGL((fwd_decode_kernel<HD, false, _Float16>), grid, dim3(256), 0, stream, d, (int)nblocks);
  } else {
    if (p.alibi) hipLaunchKernelGGL((fwd_decode_kernel<HD, true, __bf16>), grid, dim3(256), 0, stream, d, (int)nblocks);
    else hipLaunchKernelGGL((fwd_decode_kernel<HD, false, __bf16>), grid, dim3(256), 0, stream, d, (int)nblocks);
  }
  return hipGetLastError();
}
hipError_t launch_fwd_decode_d64(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_decode_d128(const FwdParams& p, hipStream_t stream);

}  // namespace fa
