// fa_fwd_kernel.hip - matrix-core (MFMA) attention forward for gfx950.
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
//  * key tiles of 64 rows are staged through LDS, double buffered, with one
//    barrier per tile; the global loads of tile t+1 are in flight while tile t
//    is computed;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    every lane then owns one query column, so the softmax row statistics are
//    lane-local plus one v_permlane32_swap between the two half-waves;
//  * K rows are stored in LDS with bits 2 and 3 of the row index swapped; with
//    that order the fp32 S^T accumulator, rounded to bf16, is already laid out as
//    the B operand of the second product O^T += V^T P^T, so P never leaves the
//    registers;
//  * V is transposed once, in registers, on its way into LDS (V^T rows of 64 keys)
//    so the A operand of O^T += V^T P^T is a plain 16-byte LDS read;
//  * exponentials use exp2 with scale*log2(e) folded into one FMA; only tiles that
//    straddle a mask boundary evaluate the per-element visibility test.
#include "fa_common.h"

namespace fa {

constexpr int BR = 128;       // query rows per workgroup
constexpr int BC = 64;        // keys per tile
constexpr int NTHREADS = 256; // 4 waves
constexpr int PAD = 8;        // bf16 padding per LDS row (16 bytes) against bank conflicts

template <int HD>
struct Tile {
  static constexpr int KROW = HD + PAD;   // K tile row pitch in LDS (elements)
  static constexpr int VROW = BC + PAD;   // V^T tile row pitch in LDS (elements)
  static constexpr int KELEMS = BC * KROW;
  static constexpr int VELEMS = HD * VROW;
  static constexpr int LDS_ELEMS = 2 * (KELEMS + VELEMS);  // two buffers
  static constexpr int CPR = HD / 8;      // 16-byte chunks per K/V row
  static constexpr int KU = BC * CPR / NTHREADS;  // K chunks per thread (= HD/32)
  static constexpr int KR = HD / 32;      // V rows per thread (one 8-wide column chunk)
  static constexpr int KB = BC / KR;      // V key blocks across the tile
};

template <int HD>
struct TileRegs {
  u32x4 k[Tile<HD>::KU];
  u32x4 v[Tile<HD>::KR];
};

// LDS row that holds key `row` of the tile: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int k_lds_row(int row) {
  return (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);
}

template <int HD>
__device__ __forceinline__ void load_tile(TileRegs<HD>& r, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, long row_stride,
                                          int j0, int key_hi, int tid) {
  using T = Tile<HD>;
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < T::KU; ++u) {
    const int id = tid + NTHREADS * u;
    const int row = id / T::CPR, col = id % T::CPR;
    const int key = j0 + row;
    r.k[u] = key < key_hi ? *(const u32x4*)(kbase + (long)key * row_stride + col * 8) : zero;
  }
  const int kb = tid % T::KB, dc = tid / T::KB;
#pragma unroll
  for (int rr = 0; rr < T::KR; ++rr) {
    const int key = j0 + kb * T::KR + rr;
    r.v[rr] = key < key_hi ? *(const u32x4*)(vbase + (long)key * row_stride + dc * 8) : zero;
  }
}

// Two bf16 halves (`half` 0 = low, 1 = high) of a and b, packed a-first.
__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, int half) {
  return half == 0 ? ((a & 0xffffu) | (b << 16)) : ((a >> 16) | (b & 0xffff0000u));
}

template <int HD>
__device__ __forceinline__ void store_tile(const TileRegs<HD>& r, uint16_t* ks, uint16_t* vt, int tid) {
  using T = Tile<HD>;
#pragma unroll
  for (int u = 0; u < T::KU; ++u) {
    const int id = tid + NTHREADS * u;
    const int row = id / T::CPR, col = id % T::CPR;
    *(u32x4*)(ks + k_lds_row(row) * T::KROW + col * 8) = r.k[u];
  }
  // V^T: this thread holds KR consecutive keys x 8 consecutive columns; write each
  // column as KR consecutive keys of one V^T row.
  const int kb = tid % T::KB, dc = tid / T::KB;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint16_t* dst = vt + (dc * 8 + d) * T::VROW + kb * T::KR;
    const int w = d >> 1, half = d & 1;
    if constexpr (T::KR == 2) {
      *(uint32_t*)dst = pick_pair(r.v[0][w], r.v[1][w], half);
    } else if constexpr (T::KR == 4) {
      u32x2 o = {pick_pair(r.v[0][w], r.v[1][w], half), pick_pair(r.v[2][w], r.v[3][w], half)};
      *(u32x2*)dst = o;
    } else {
      u32x4 o = {pick_pair(r.v[0][w], r.v[1][w], half), pick_pair(r.v[2][w], r.v[3][w], half),
                 pick_pair(r.v[4][w], r.v[5][w], half), pick_pair(r.v[6][w], r.v[7][w], half)};
      *(u32x4*)dst = o;
    }
  }
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
  const uint16_t* __restrict__ kbase = p.k + (long)b * Sk * row_stride + (long)h * HD;
  const uint16_t* __restrict__ vbase = p.v + (long)b * Sk * row_stride + (long)h * HD;

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
  const int my_q = i0 + wave * 32 + lrow;
  const int my_pos = my_q + off;
  bf16x8 qf[HD / 16];
#pragma unroll
  for (int kk = 0; kk < HD / 16; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (my_q < Sq) raw = *(const u32x4*)(qbase + (long)my_q * row_stride + 16 * kk + 8 * half);
    raw ^= p.q_sign;
    qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int db = 0; db < HD / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 units
  float l_run = 0.f;        // this lane's share of the running row sum
  const float c = p.scale_log2;
  float slope = 0.f;
  if constexpr (ALIBI) slope = p.alibi[h] * kLog2e;  // bias in log2 units

  TileRegs<HD> regs;
  int buf = 0;
  if (t_begin < t_end) {
    load_tile<HD>(regs, kbase, vbase, row_stride, key_lo + t_begin * BC, key_hi, tid);
    store_tile<HD>(regs, ks0, vt0, tid);
    __syncthreads();
  }

  for (int t = t_begin; t < t_end; ++t) {
    const int j0 = key_lo + t * BC;
    const bool has_next = t + 1 < t_end;
    if (has_next) load_tile<HD>(regs, kbase, vbase, row_stride, j0 + BC, key_hi, tid);

    const uint16_t* kt = ks0 + buf * T::KELEMS;
    const uint16_t* vtile = vt0 + buf * T::VELEMS;

    // S^T (64 keys x 32 queries per wave) as two 32x32 blocks.
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kt + (32 * kb + lrow) * T::KROW + 16 * kk + 8 * half);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kb], 0, 0, 0);
      }
    }

    // Is every (row, key) of this tile visible to every valid row of the block?
    const bool full = (j0 + BC <= key_hi) && (wl < 0 || j0 >= i_last + off - wl) &&
                      (wr < 0 || j0 + BC - 1 <= i0 + off + wr);

    float tmax;
    if (ALIBI || !full) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // key held by (lane, r): see k_lds_row for the row order
          const int key = j0 + 32 * kb + 16 * (r >> 3) + 8 * half + (r & 7);
          float tv = s[kb][r] * c;
          if constexpr (ALIBI) tv -= slope * fabsf((float)(my_pos - key));
          if (!full) {
            const bool vis = key < key_hi && (wl < 0 || key >= my_pos - wl) && (wr < 0 || key <= my_pos + wr);
            tv = vis ? tv : -INFINITY;
          }
          s[kb][r] = tv;
          mx = fmaxf(mx, tv);
        }
      }
      tmax = max_with_other_half(mx);
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      tmax = max_with_other_half(mx) * c;
    }

    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // empty so far: keep exp args finite
    const float alpha = fast_exp2(m_run - m_use);
    float rsum = 0.f;
    if (ALIBI || !full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(s[kb][r] - m_use);
          s[kb][r] = pv;
          rsum += pv;
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(fmaf(s[kb][r], c, -m_use));
          s[kb][r] = pv;
          rsum += pv;
        }
    }
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    // P^T in bf16: chunk ci (16 keys) is the B operand of one 32x32x16 product.
    bf16x8 pf[4];
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) {
      const f32x16& src = s[ci >> 1];
      const int r0 = 8 * (ci & 1);
      u32x4 pk = {pack_bf16x2(src[r0 + 0], src[r0 + 1]), pack_bf16x2(src[r0 + 2], src[r0 + 3]),
                  pack_bf16x2(src[r0 + 4], src[r0 + 5]), pack_bf16x2(src[r0 + 6], src[r0 + 7])};
      pf[ci] = __builtin_bit_cast(bf16x8, pk);
    }

    // O^T (HD x 32 queries) += V^T P^T
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) {
#pragma unroll
      for (int ci = 0; ci < 4; ++ci) {
        const bf16x8 a = *(const bf16x8*)(vtile + (32 * db + lrow) * T::VROW + 16 * ci + 8 * half);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ci], oacc[db], 0, 0, 0);
      }
    }

    if (has_next) store_tile<HD>(regs, ks0 + (buf ^ 1) * T::KELEMS, vt0 + (buf ^ 1) * T::VELEMS, tid);
    __syncthreads();
    buf ^= 1;
  }

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
static hipError_t launch(const FwdParams& p, long nblocks, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<HD, ALIBI, SPLIT>), dim3((unsigned)nblocks), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

template <bool ALIBI, bool SPLIT>
static hipError_t launch_hd(const FwdParams& p, int headdim, long nblocks, hipStream_t stream) {
  switch (headdim) {
    case 64: return launch<64, ALIBI, SPLIT>(p, nblocks, stream);
    case 128: return launch<128, ALIBI, SPLIT>(p, nblocks, stream);
    case 256: return launch<256, ALIBI, SPLIT>(p, nblocks, stream);
    default: return hipErrorInvalidValue;
  }
}

// Host-side launcher used by the C ABI layer.  Arguments are already validated.
hipError_t launch_fwd(const FwdParams& p, int headdim, bool split, hipStream_t stream) {
  const long nblocks = (long)p.batch * p.nheads * p.num_q_tiles * (split ? p.num_splits : 1);
  const bool alibi = p.alibi != nullptr;
  if (split) return alibi ? launch_hd<true, true>(p, headdim, nblocks, stream)
                          : launch_hd<false, true>(p, headdim, nblocks, stream);
  return alibi ? launch_hd<true, false>(p, headdim, nblocks, stream)
               : launch_hd<false, false>(p, headdim, nblocks, stream);
}

long fwd_num_blocks(const FwdParams& p, bool split) {
  return (long)p.batch * p.nheads * p.num_q_tiles * (split ? p.num_splits : 1);
}

}  // namespace fa
