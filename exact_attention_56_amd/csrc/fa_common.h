// fa_common.h - device types and small helpers shared by the gfx950 attention
// kernels (the parameter blocks are in fa_params.h).  Internal to the library (not
// part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_params.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// q, k, v, out (and the gradients) are bf16 or fp16: the same 16-bit storage, so
// loads, LDS layouts and address arithmetic are shared; the element type E
// (__bf16 or _Float16) only picks the matrix-core instruction, the rounding of fp32
// results to 16 bits and the widening to fp32.
template <typename E>
using x8 = E __attribute__((ext_vector_type(8)));
template <typename E>
using x2 = E __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x in lane (l ^ 32) combined with x by a symmetric operation: both
// halves of the wave exchange their values with one v_permlane32_swap.
__device__ __forceinline__ float max_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round two fp32 to bf16 (round-to-nearest-even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// 32x32x16 matrix-core product with fp32 accumulation, for either element type.
__device__ __forceinline__ f32x16 mfma32(const x8<__bf16>& a, const x8<__bf16>& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const x8<_Float16>& a, const x8<_Float16>& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Round two fp32 to E (round-to-nearest-even) and pack them, low half first.
template <typename E>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, x2<E>));
}

// fp32 value of the low / high 16-bit element of a packed pair.
template <typename E>
__device__ __forceinline__ float widen_lo(uint32_t x) {
  if constexpr (__is_same(E, __bf16)) return __uint_as_float(x << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
}
template <typename E>
__device__ __forceinline__ float widen_hi(uint32_t x) {
  if constexpr (__is_same(E, __bf16)) return __uint_as_float(x & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}

// Map a linear workgroup id to a work index so that the workgroups the dispatcher
// sends to one XCD (ids congruent mod 8) receive one contiguous range of work
// indices: neighbouring query tiles of one (batch, head) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int per = nblocks >> 3;
  const int rem = nblocks & 7;
  return (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Launches whose tiles differ in length (causal mask or right window): item w of an
// XCD-contiguous order (w = xcd_remap(...)) over (pair, tile), pairs = batch * nheads.
// Pairs form groups of up to four (at most one XCD's share, whose K/V then stays in
// that XCD's L2 while the group runs); inside a group the tile index runs slowest, so
// the heaviest tiles of every pair start first and short ones fill the end.  Returns
// the pair; `rank` gets the tile's position in the group's order (0 first).
__device__ __forceinline__ int heavy_first_item(int w, int ntiles, int pairs, int& rank) {
  const int gsize = min(4, max(1, pairs / 8));
  const int group = w / (gsize * ntiles);
  const int r = w % (gsize * ntiles);
  const int gp = min(gsize, pairs - group * gsize);  // pairs in this group (the last may be short)
  rank = r / gp;
  return group * gsize + r % gp;
}

}  // namespace fa
