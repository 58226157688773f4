// Helpers shared by the sparse-attention kernels (forward, backward, KL objective): block
// shape, bf16 rounding and loads, cross-row reductions, the transposing LDS read and the
// bank swizzle of staged K/V rows.
#pragma once

#include "ix_common.h"

namespace ix {

constexpr int kAttnWaves = 4;
constexpr int kAttnBlock = kAttnWaves * kWave;
constexpr int kChunk = 32;


// Two floats to packed bf16 (lo in bits 0-15), rounded to nearest even by the gfx950
// conversion instruction (one instruction for the pair; NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// One float to bf16 bits, rounded to nearest even (the same conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// 2^x by the hardware instruction alone: exact to its rounding for results of 2^-126 and up;
// below that (a softmax weight under 2^-126 of the running maximum, far below what a bf16
// output or an fp32 sum of such weights can show) it need not give the denormal.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

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

// bf16 16x16x16: D += A(16x16) * B(16x16); lane l supplies A[l & 15][4(l>>4) .. +3] and
// B[4(l>>4) .. +3][l & 15].
__device__ __forceinline__ f32x4 mfma_bf16_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane i receives element (i & 3) of
// the 8-byte reads of lanes 4r + (i >> 2), r = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// Bank swizzle of the staged K/V rows: 16-byte piece p of chunk slot n sits at piece
// position p ^ swz(n).  D = 128 (256-byte rows): swz(n) over n mod 16 is the permutation
// 0 2 4 6 9 11 13 15 1 3 5 7 8 10 12 14, so that the 16 slots of an A-operand read (16 bytes
// per lane) take 16 distinct 16-byte positions and each 8 of them distinct positions modulo 8,
// the slots of a transposed read (8 bytes per lane) distinct 8-byte positions per 32 and per
// 16 lanes, and a row's 16 pieces written by 16 lanes distinct positions per 16 and per 8
// lanes: no bank conflict whether a 16-byte access serves 8 or 16 lanes per cycle.  (A plain
// one-bit rotation gave the A-operand reads two-way conflicts in the 8-lane case.)  D = 64
// (128-byte rows, two per 256 bytes): the slot pair's position rotated left by one bit.
template <int D>
__device__ __forceinline__ int stage_swz(int n) {
  if constexpr (D == 128) {
    const int m = n & 15;
    return (2 * (m & 3)) | (((m >> 2) & 1) << 3) | (((m >> 2) ^ (m >> 3)) & 1);
  } else {
    const int m = (n >> 1) & 7;
    return ((m << 1) & 7) | (m >> 2);
  }
}

}  // namespace ix
