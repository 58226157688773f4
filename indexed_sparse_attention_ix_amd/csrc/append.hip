// Cache append: the producer side of the FP8 indexer-key cache and the K/V caches, the
// step just before Stage 1 ("GLM 5.2: How Four Co-Designed Mechanisms Beat Raw Scale",
// Part II, "DeepSeek Sparse Attention") in a decode loop.  The indexer runs in FP8 (the
// twiscan post on GLM-5.2's IndexShare); new indexer keys are rounded to OCP e4m3 here:
// clamped to +-448 (the largest finite e4m3 magnitude), then rounded to nearest, ties to
// even, by the hardware conversion.  New bf16 K/V rows are copied unchanged.
//
// Both kernels are plain streaming copies: one thread per 8 key elements (two 16-byte
// loads, one 8-byte store) and one thread per 16 bytes of a K or V row.  Rows whose
// position pos0[b] + t falls outside [0, S_max) are skipped.
#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

constexpr int kAppendBlock = 256;

// Clamp to the largest finite e4m3 magnitude; NaN passes through (fmaxf/fminf would
// replace it by the bound).
__device__ __forceinline__ float clamp448(float x) {
  const float c = fminf(fmaxf(x, -448.f), 448.f);
  return x != x ? x : c;
}

// Two fp32 values -> two e4m3 bytes in the low half of the result (v_cvt_pk_fp8_f32,
// round to nearest even).  The clamp keeps the conversion away from its overflow path.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false) & 0xFFFFu;
}

__global__ __launch_bounds__(kAppendBlock) void append_keys_kernel(
    const float* __restrict__ kn, const int32_t* __restrict__ pos0, int B, int T, int S_max,
    int DI, uint8_t* __restrict__ kc) {
  const int64_t gid = (int64_t)blockIdx.x * kAppendBlock + threadIdx.x;
  const int per_row = DI / 8;
  const int64_t row = gid / per_row;  // b * T + t
  if (row >= (int64_t)B * T) return;
  const int part = (int)(gid - row * per_row);
  const int b = (int)(row / T), t = (int)(row - (int64_t)b * T);
  const int64_t pos = (int64_t)pos0[b] + t;
  if (pos < 0 || pos >= S_max) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(kn + row * DI + 8 * part);
  const f32x4 lo = src[0], hi = src[1];
  uint2 out;
  out.x = e4m3_pair(lo[0], lo[1]) | (e4m3_pair(lo[2], lo[3]) << 16);
  out.y = e4m3_pair(hi[0], hi[1]) | (e4m3_pair(hi[2], hi[3]) << 16);
  *reinterpret_cast<uint2*>(kc + ((int64_t)b * S_max + pos) * DI + 8 * part) = out;
}

// One thread per 16-byte piece of a (token, KV head) row of K and of V.
__global__ __launch_bounds__(kAppendBlock) void append_kv_rows_kernel(
    const uint16_t* __restrict__ Kn, const uint16_t* __restrict__ Vn,
    const int32_t* __restrict__ pos0, int B, int T, int S_max, int row_elems,
    uint16_t* __restrict__ Kc, uint16_t* __restrict__ Vc) {
  const int64_t gid = (int64_t)blockIdx.x * kAppendBlock + threadIdx.x;
  const int per_row = row_elems / 8;  // H_kv * d bf16 values per token
  const int64_t row = gid / per_row;
  if (row >= (int64_t)B * T) return;
  const int part = (int)(gid - row * per_row);
  const int b = (int)(row / T), t = (int)(row - (int64_t)b * T);
  const int64_t pos = (int64_t)pos0[b] + t;
  if (pos < 0 || pos >= S_max) return;
  const int64_t src = row * row_elems + 8 * part;
  const int64_t dst = ((int64_t)b * S_max + pos) * row_elems + 8 * part;
  if (Kc) *reinterpret_cast<i32x4*>(Kc + dst) = *reinterpret_cast<const i32x4*>(Kn + src);
  if (Vc) *reinterpret_cast<i32x4*>(Vc + dst) = *reinterpret_cast<const i32x4*>(Vn + src);
}

}  // namespace

hipError_t launch_append_kv(const float* k_I_new, const void* K_new, const void* V_new,
                            const int32_t* pos0, int B, int T_new, int S_max, int d_I, int H_kv,
                            int d, uint8_t* k_I_cache, void* K_cache, void* V_cache,
                            hipStream_t stream) {
  const int64_t rows = (int64_t)B * T_new;
  if (k_I_new) {
    const int64_t threads = rows * (d_I / 8);
    hipLaunchKernelGGL(append_keys_kernel, dim3((unsigned)((threads + kAppendBlock - 1) / kAppendBlock)),
                       dim3(kAppendBlock), 0, stream, k_I_new, pos0, B, T_new, S_max, d_I, k_I_cache);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (K_new || V_new) {
    const int row_elems = H_kv * d;
    const int64_t threads = rows * (row_elems / 8);
    hipLaunchKernelGGL(append_kv_rows_kernel,
                       dim3((unsigned)((threads + kAppendBlock - 1) / kAppendBlock)),
                       dim3(kAppendBlock), 0, stream, reinterpret_cast<const uint16_t*>(K_new),
                       reinterpret_cast<const uint16_t*>(V_new), pos0, B, T_new, S_max, row_elems,
                       reinterpret_cast<uint16_t*>(K_cache), reinterpret_cast<uint16_t*>(V_cache));
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace ix
