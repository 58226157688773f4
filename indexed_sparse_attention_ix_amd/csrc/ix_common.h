// Device helpers shared by the gfx950 kernels: MFMA wrappers, DPP lane exchanges,
// order-preserving float <-> integer keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ix {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// One 16x16 output tile of an FP8 (OCP e4m3) product with depth 128:
// D[i][j] = sum_k A[i][k] * B[j][k], fp32.  Lane l supplies row (l & 15) of A and of B
// as 32 bytes; the four lane groups (l >> 4) supply the four 32-byte slices of the
// depth.  D comes back as lane l holding D[4*(l>>4) + r][l & 15], r = 0..3.
// Zero scale operands select the unscaled v_mfma_f32_16x16x128_f8f6f4.
__device__ __forceinline__ f32x4 mfma_e4m3_16x16x128(i32x8 a, i32x8 b) {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// bf16 16x16x32: D += A(16x32) * B(32x16); lane l supplies row/col (l & 15) and the
// depth slice [8*(l>>4), 8*(l>>4)+8).
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;  // row_ror:4
constexpr int kDppRowRor8 = 0x128;  // row_ror:8

template <int Ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), Ctrl, 0xF, 0xF, true));
}

// Order-preserving map fp32 -> uint32 (larger float -> larger integer); -0 is first
// folded onto +0 so both zeros share one key.
__device__ __forceinline__ uint32_t f32_to_ordered(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float ordered_to_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}
__device__ __forceinline__ int popc64(uint64_t x) { return __builtin_popcountll(x); }
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

template <typename T>
__device__ __forceinline__ T readlane(T v, int lane) {
  return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Wait for this wave's outstanding LDS operations.
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Wait for this wave's outstanding vector-memory operations.
__device__ __forceinline__ void vmem_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cache-policy operand of a buffer load that marks it non-temporal (data read once).
constexpr int kLoadNT = 2;

// Raw buffer resource over `bytes` bytes at `base`: loads at offsets >= bytes return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ i32x4 ld_global_16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}

}  // namespace ix
