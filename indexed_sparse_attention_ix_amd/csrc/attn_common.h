// Helpers shared by the sparse-attention kernels (forward, backward, KL objective): block
// shape, bf16 rounding and loads, cross-row reductions, the transposing LDS read and the
// bank swizzle of staged K/V rows.
#pragma once

#include "ix_common.h"

namespace ix {

constexpr int kAttnWaves = 4;
constexpr int kAttnBlock = kAttnWaves * kWave;
constexpr int kChunk = 32;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, ld_global_16(p));
}

// Reductions across the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48).
// v_permlane16_swap x, y exchanges x's rows 1, 3 with y's rows 0, 2 (v_permlane32_swap:
// x's upper half with y's lower half).  With y a copy of x, x and y then hold each row
// and its neighbour, so one max/add per stage pairs the rows.  Written as asm with both
// registers read-write: the compiler's model of the builtin drops one of the two
// results when the operands are equal.  The s_nop's give the VALU <-> permlane hazard
// its wait states.
__device__ __forceinline__ void row_pair_swap16(uint32_t& x, uint32_t& y) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void row_pair_swap32(uint32_t& x, uint32_t& y) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ float max_across_rows(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  row_pair_swap16(x, y);
  v = fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
  x = y = __builtin_bit_cast(uint32_t, v);
  row_pair_swap32(x, y);
  return fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}
__device__ __forceinline__ float sum_across_rows(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  row_pair_swap16(x, y);
  v = __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
  x = y = __builtin_bit_cast(uint32_t, v);
  row_pair_swap32(x, y);
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}

// Transposing LDS read: within each 16-lane group, lane i receives element (i & 3) of
// the 8-byte reads of lanes 4r + (i >> 2), r = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// Bank swizzle of the staged K/V rows: 16-byte piece p of chunk slot n sits at piece
// position p ^ swz(n).  Rows are 256 B (D = 128: one row per 64-bank line) or 128 B
// (D = 64: two rows per line); swz rotates the slot's position within the line left by
// one bit, so the 16 slots of an A-operand read hit 16 distinct 16-byte bank groups and
// the 8 slots of a half-wave transposed read hit 8 distinct 32-byte groups.
template <int D>
__device__ __forceinline__ int stage_swz(int n) {
  constexpr int PI = D / 8;                     // 16-byte pieces per row
  constexpr int LOG = D == 128 ? 4 : 3;
  const int m = (D == 128 ? n : (n >> 1)) & (PI - 1);
  return ((m << 1) & (PI - 1)) | (m >> (LOG - 1));
}

}  // namespace ix
