// Measured ceilings for the roofline fractions: what gfx950 delivers on the three shapes of
// work the path is made of, next to the datasheet peaks.
//  * FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4) issued back to back, alone or followed by
//    N fp32 VALU ops per MFMA -- the indexer spends 8 per MFMA on its epilogue (an integer
//    max and an FMA per output element), so N = 8 is the rate its core can reach.
//  * a device copy with 16-byte loads and stores (the HBM stream rate);
//  * gathers of whole 256-byte rows at random from a table (the attention's access
//    pattern: a bf16 K or V row at d = 128), read by 16 consecutive lanes per row;
//  * fp32 atomic adds of whole 128-float rows at random rows of a table (the attention
//    backward's dK/dV accumulation: one row per selected key, two 64-lane instructions).
// None of these kernels touches memory outside the caller's buffers.
#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

constexpr int kPeakBlock = 256;
constexpr int kPeakHeads = 16;  // B operands held in registers, as in the indexer

__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

template <int NV>
__device__ __forceinline__ void peak_epilogue(f32x4& acc, const f32x4& x, float w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = x[i];
    if constexpr (NV >= 8) v = relu_bits(v);
    acc[i] = fmaf(w, v, acc[i]);
    if constexpr (NV >= 12) acc[i] = acc[i] * 0.999f;
  }
}

// Each iteration: one A tile (loaded one iteration ahead, like the indexer's key tiles)
// against the 16 register-resident B operands.  NV > 0: the epilogue of MFMA g-2 follows
// the issue of MFMA g (two in flight, so no dependent stall); NV = 0: results feed the
// accumulator of MFMA g+2.
template <int NV>
__global__ __launch_bounds__(kPeakBlock, 2) void peak_mfma_kernel(const i32x8* __restrict__ tab,
                                                                  int iters, float* __restrict__ out) {
  const int l = threadIdx.x & 63;
  i32x8 b[kPeakHeads];
  float w[kPeakHeads];
#pragma unroll
  for (int g = 0; g < kPeakHeads; ++g) {
    b[g] = tab[64 * (g + 1) + l];
    w[g] = 0.5f + 0.01f * g;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 c0 = acc, c1 = acc;
  i32x8 a_next = tab[l];
  for (int it = 0; it < iters; ++it) {
    const i32x8 a = a_next;  // this tile's A; the next one loads under its MFMAs
    a_next = tab[((it + 1) & 1) * 64 * (kPeakHeads + 1) + l];
    if constexpr (NV == 0) {
#pragma unroll
      for (int g = 0; g < kPeakHeads; g += 2) {
        c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[g], c0, 0, 0, 0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[g + 1], c1, 0, 0, 0, 0, 0, 0);
      }
    } else {
      f32x4 x0 = mfma_e4m3_16x16x128(a, b[0]);
      f32x4 x1 = mfma_e4m3_16x16x128(a, b[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 2; g < kPeakHeads; ++g) {
        const f32x4 y = mfma_e4m3_16x16x128(a, b[g]);
        peak_epilogue<NV>(acc, x0, w[g - 2]);
        x0 = x1;
        x1 = y;
        __builtin_amdgcn_sched_barrier(0);
      }
      peak_epilogue<NV>(acc, x0, w[kPeakHeads - 2]);
      peak_epilogue<NV>(acc, x1, w[kPeakHeads - 1]);
    }
  }
  float v = acc[0] + acc[1] + acc[2] + acc[3] + c0[0] + c0[1] + c0[2] + c0[3] + c1[0] + c1[1] +
            c1[2] + c1[3];
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if (l == 0) atomicAdd(out, v);
}

__global__ __launch_bounds__(kPeakBlock) void peak_copy_kernel(const i32x4* __restrict__ src,
                                                               i32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kPeakBlock;
  for (int64_t i = (int64_t)blockIdx.x * kPeakBlock + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Rows of 256 bytes: lane piece s = lane % 16 of row rows[r], four rows per load
// instruction, 16 loads in flight per lane.  The table is read through a buffer resource
// whose size bounds every access (an out-of-range row reads as zero).
constexpr int kGatherInFlight = 16;

__global__ __launch_bounds__(kPeakBlock) void peak_gather_kernel(const void* __restrict__ table,
                                                                 uint32_t table_bytes,
                                                                 const int32_t* __restrict__ rows,
                                                                 int64_t n, uint32_t* __restrict__ out) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(table, table_bytes);
  const int lane = threadIdx.x & 63;
  const int s = lane & 15;
  const int64_t group = ((int64_t)blockIdx.x * kPeakBlock + threadIdx.x) >> 4;
  const int64_t groups = ((int64_t)gridDim.x * kPeakBlock) >> 4;
  uint32_t x = 0;
  for (int64_t base = group; base < n; base += groups * kGatherInFlight) {
    i32x4 v[kGatherInFlight];
#pragma unroll
    for (int j = 0; j < kGatherInFlight; ++j) {
      const int64_t r = base + (int64_t)j * groups;
      const uint32_t off = r < n ? (uint32_t)rows[r] * 256u + 16u * s : 0x80000000u;
      v[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < kGatherInFlight; ++j) x ^= (uint32_t)(v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3]);
  }
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  if (lane == 0) atomicXor(out, x);
}

// One listed row per wave and step: lanes add 1 to floats [0, 64) and [64, 128) of the row
// (the row index is wave-uniform); rows outside [0, rows) are skipped.
__global__ __launch_bounds__(kPeakBlock) void peak_atomic_kernel(float* __restrict__ table, int64_t rows,
                                                                 const int32_t* __restrict__ idx,
                                                                 int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kPeakBlock + threadIdx.x) >> 6;
  const int64_t waves = ((int64_t)gridDim.x * kPeakBlock) >> 6;
  for (int64_t e = wave; e < n; e += waves) {
    const int r = __builtin_amdgcn_readfirstlane(idx[e]);
    if (r < 0 || r >= rows) continue;
    float* row = table + (int64_t)r * 128;
    atomicAdd(row + lane, 1.f);
    atomicAdd(row + 64 + lane, 1.f);
  }
}

}  // namespace

hipError_t launch_peak_atomic(float* table, int64_t rows, const int32_t* idx, int64_t n,
                              hipStream_t stream) {
  hipLaunchKernelGGL(peak_atomic_kernel, dim3(256 * 8), dim3(kPeakBlock), 0, stream, table, rows,
                     idx, n);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(const void* operands, int valu_per_mfma, int blocks, int iters,
                            float* out, hipStream_t stream) {
  const i32x8* tab = reinterpret_cast<const i32x8*>(operands);
  const dim3 g((unsigned)blocks), b(kPeakBlock);
  switch (valu_per_mfma) {
    case 0: hipLaunchKernelGGL(peak_mfma_kernel<0>, g, b, 0, stream, tab, iters, out); break;
    case 4: hipLaunchKernelGGL(peak_mfma_kernel<4>, g, b, 0, stream, tab, iters, out); break;
    case 8: hipLaunchKernelGGL(peak_mfma_kernel<8>, g, b, 0, stream, tab, iters, out); break;
    default: hipLaunchKernelGGL(peak_mfma_kernel<12>, g, b, 0, stream, tab, iters, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(peak_copy_kernel, dim3(256 * 16), dim3(kPeakBlock), 0, stream,
                     reinterpret_cast<const i32x4*>(src), reinterpret_cast<i32x4*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_peak_gather(const void* table, size_t table_bytes, const int32_t* rows, int64_t n,
                              uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(peak_gather_kernel, dim3(256 * 8), dim3(kPeakBlock), 0, stream, table,
                     (uint32_t)table_bytes, rows, n, out);
  return hipGetLastError();
}

}  // namespace ix
