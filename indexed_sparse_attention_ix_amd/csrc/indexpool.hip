// IndexPool (GLM-5.3-Flash as recorded on worldresearchstate.com, "What changed": four
// indexer keys are pooled into one to cut the cost of long-context indexing).  The page
// gives no more than that; the reading implemented here:
//  * a block key is the mean of `pool` consecutive tokens' FP8 indexer keys, rounded to
//    e4m3 (nearest, ties to even); tokens at or past kv_len count as zero, so every block
//    divides by `pool` and the mean is exact in fp32 before the rounding;
//  * the fused indexer + top-k runs unchanged over block keys, a query at position p
//    seeing block j once pool*j <= p;
//  * each kept block expands to its `pool` token positions, those the query does not see
//    becoming -1 (only the last kept block can be cut short), so rows stay ascending
//    with the padding at the end.
#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

constexpr int kPoolBlock = 256;

__device__ __forceinline__ float clamp448(float x) {
  const float c = fminf(fmaxf(x, -448.f), 448.f);
  return x != x ? x : c;
}

// One thread per 8 elements of one block key: decode the block's e4m3 rows, sum and
// divide by pool.  A sum of at most 16 e4m3 values is exact in fp32 (multiples of 2^-9
// below 2^13) and pool is a power of two, so the mean is exact before it is rounded back
// to e4m3.
__global__ __launch_bounds__(kPoolBlock) void pool_keys_kernel(const uint8_t* __restrict__ k,
                                                               const int32_t* __restrict__ kv_len,
                                                               int B, int S_max, int DI, int pool,
                                                               int S_blocks,
                                                               uint8_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * kPoolBlock + threadIdx.x;
  const int per_row = DI / 8;
  const int64_t row = gid / per_row;  // b * S_blocks + j
  if (row >= (int64_t)B * S_blocks) return;
  const int part = (int)(gid - row * per_row);
  const int b = (int)(row / S_blocks), j = (int)(row - (int64_t)b * S_blocks);
  int kvl = kv_len ? kv_len[b] : S_max;
  kvl = kvl < 0 ? 0 : (kvl > S_max ? S_max : kvl);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < pool; ++r) {
    const int s = pool * j + r;
    if (s >= kvl) break;
    const uint2 v = *reinterpret_cast<const uint2*>(k + ((int64_t)b * S_max + s) * DI + 8 * part);
    const uint32_t w[2] = {v.x, v.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], true);
      acc[4 * h + 0] += lo[0];
      acc[4 * h + 1] += lo[1];
      acc[4 * h + 2] += hi[0];
      acc[4 * h + 3] += hi[1];
    }
  }
  const float inv = 1.0f / (float)pool;  // exact: pool is a power of two
  uint32_t o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
        clamp448(acc[4 * h] * inv), clamp448(acc[4 * h + 1] * inv), 0, false) & 0xFFFFu;
    const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
        clamp448(acc[4 * h + 2] * inv), clamp448(acc[4 * h + 3] * inv), 0, false) & 0xFFFFu;
    o[h] = a | (c << 16);
  }
  *reinterpret_cast<uint2*>(out + row * DI + 8 * part) = make_uint2(o[0], o[1]);
}

// One thread per output entry: entry e of row (b, t) is token pool*j + e % pool of kept
// block j = blocks[b, t, e / pool], or -1 when there is no such block or the query does
// not see that token.
__global__ __launch_bounds__(kPoolBlock) void expand_blocks_kernel(
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ q_pos0,
    const int32_t* __restrict__ kv_len, int B, int T, int S_max, int k_blocks, int pool,
    int32_t* __restrict__ idx) {
  const int64_t gid = (int64_t)blockIdx.x * kPoolBlock + threadIdx.x;
  const int64_t width = (int64_t)k_blocks * pool;
  const int64_t row = gid / width;  // b * T + t
  if (row >= (int64_t)B * T) return;
  const int e = (int)(gid - row * width);
  const int b = (int)(row / T), t = (int)(row - (int64_t)b * T);
  int kvl = kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > S_max ? S_max : kvl);
  const int64_t p1 = (int64_t)q_pos0[b] + t + 1;
  const int n_t = (int)(p1 < 0 ? 0 : (p1 > kvl ? kvl : p1));
  const int j = blocks[row * k_blocks + e / pool];
  const int64_t tok = (int64_t)pool * j + e % pool;
  idx[gid] = (j >= 0 && tok < n_t) ? (int32_t)tok : -1;
}

}  // namespace

hipError_t launch_pool_keys(const uint8_t* k_I, const int32_t* kv_len, int B, int S_max, int d_I,
                            int pool, uint8_t* k_pooled, hipStream_t stream) {
  const int S_blocks = (S_max + pool - 1) / pool;
  const int64_t threads = (int64_t)B * S_blocks * (d_I / 8);
  hipLaunchKernelGGL(pool_keys_kernel, dim3((unsigned)((threads + kPoolBlock - 1) / kPoolBlock)),
                     dim3(kPoolBlock), 0, stream, k_I, kv_len, B, S_max, d_I, pool, S_blocks,
                     k_pooled);
  return hipGetLastError();
}

hipError_t launch_expand_blocks(const int32_t* blocks, const int32_t* q_pos0,
                                const int32_t* kv_len, int B, int T, int S_max, int k_blocks,
                                int pool, int32_t* idx, hipStream_t stream) {
  const int64_t threads = (int64_t)B * T * k_blocks * pool;
  hipLaunchKernelGGL(expand_blocks_kernel, dim3((unsigned)((threads + kPoolBlock - 1) / kPoolBlock)),
                     dim3(kPoolBlock), 0, stream, blocks, q_pos0, kv_len, B, T, S_max, k_blocks,
                     pool, idx);
  return hipGetLastError();
}

}  // namespace ix
