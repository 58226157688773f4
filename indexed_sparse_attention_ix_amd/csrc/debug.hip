// The library's debug status (ix_debug_enable / ix_debug_read): a count of the entries of a
// caller's selection that name no key.  The kernel runs only while the status is on; the
// attention kernels themselves skip such entries either way.
#include <algorithm>

#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

__global__ __launch_bounds__(256) void idx_check_kernel(const int32_t* idx, const int32_t* kv_len,
                                                        int T, int S_max, int k, int64_t n,
                                                        unsigned long long* dbg) {
  uint32_t bad = 0;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int b = (int)((e / k) / T);
    int kvl = kv_len ? kv_len[b] : S_max;
    kvl = kvl < 0 ? 0 : (kvl > S_max ? S_max : kvl);
    const int s = idx[e];
    bad += (s < -1 || s >= kvl) ? 1u : 0u;
  }
  for (int off = 32; off > 0; off >>= 1) bad += (uint32_t)__shfl_xor((int)bad, off);
  if ((threadIdx.x & 63) == 0 && bad) atomicAdd(dbg + kDbgIdxOutOfRange, (unsigned long long)bad);
}

}  // namespace

hipError_t launch_idx_check(const int32_t* idx, const int32_t* kv_len, int B, int T, int S_max,
                            int k, unsigned long long* dbg, hipStream_t stream) {
  const int64_t n = (int64_t)B * T * k;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((n + 255) / 256, 4096));
  hipLaunchKernelGGL(idx_check_kernel, grid, dim3(256), 0, stream, idx, kv_len, T, S_max, k, n, dbg);
  return hipGetLastError();
}

}  // namespace ix
