// Measured ceilings for the roofline fractions (libix_peaks.so, a library of its own: the
// path's library does not contain these kernels): what gfx950 delivers on the shapes of work
// the path is made of, next to the datasheet peaks.
//  * FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4) issued back to back, alone or followed by
//    N fp32 VALU ops per MFMA -- the indexer spends 8 per MFMA on its epilogue (an integer
//    max and an FMA per output element), so N = 8 is the rate its core can reach.
//  * a device copy and a read-only stream with 16-byte accesses (the HBM stream rates);
//  * gathers of whole 256-byte rows at random from a table, read by 16 consecutive lanes
//    per row;
//  * gathers of exactly the K and V rows a selection names, with the sparse attention's
//    block shape and block order (one block of 4 waves per query and KV head, 32-entry
//    chunks, two chunks in flight per wave, XCD-aware block numbering) and nothing computed:
//    the memory system's rate for the attention's own access pattern, including what the
//    L2 and the Infinity Cache serve;
//  * fp32 atomic adds of whole 128-float rows at random rows of a table (the attention
//    backward's dK/dV accumulation: one row per selected key, two 64-lane instructions).
// None of these kernels touches memory outside the caller's buffers.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "../../include/ix_peaks.h"
#include "../csrc/ix_common.h"

namespace ix {

namespace {

constexpr int kPeakBlock = 256;
constexpr int kPeakHeads = 16;  // B operands held in registers, as in the indexer
constexpr int kReadBlocks = 4096;    // grid of the copy kernel
constexpr int kMaxPeakBlocks = 65536;  // grids the read and gather ceilings accept

// XOR of x over the block, stored by thread 0 at out[blockIdx.x] (a plain store per block:
// no atomics on one shared word, which would serialise at one L2 channel).
__device__ __forceinline__ void block_xor_store(uint32_t x, uint32_t* out) {
  __shared__ uint32_t part[kPeakBlock / 64];
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
    for (int w = 0; w < kPeakBlock / 64; ++w) v ^= part[w];
    out[blockIdx.x] = v;
  }
}

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
// instruction, 8 loads in flight per lane (deeper queues measured slower from a 2 GiB table:
// 16 in flight 5.0-5.1 TB/s, 32 in flight 4.2, against 6.3 for 2 to 8).  No non-temporal
// hint: it costs 15 % when the table sits in the Infinity Cache (8.5 -> 7.3 TB/s from 64 MiB)
// and gains 2.5 % from HBM.  The table is n_seg segments of seg_bytes, each read through a
// buffer resource whose size bounds every access (an out-of-range row reads as zero); load
// step i of wave w reads in segment (w + i) mod n_seg, so a footprint past the 32-bit offsets
// of one resource is spread over the whole grid.
constexpr int kGatherInFlight = 8;

template <int AUX>
__global__ __launch_bounds__(kPeakBlock) void peak_gather_kernel(const unsigned char* __restrict__ table,
                                                                 uint32_t seg_bytes, int n_seg,
                                                                 const int32_t* __restrict__ rows,
                                                                 int64_t n, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int s = lane & 15;
  const int64_t tid = (int64_t)blockIdx.x * kPeakBlock + threadIdx.x;
  const int64_t wave = tid >> 6;
  const int64_t group = tid >> 4;
  const int64_t groups = ((int64_t)gridDim.x * kPeakBlock) >> 4;
  uint32_t x = 0;
  int64_t step = 0;
  for (int64_t base = group; base < n; base += groups * kGatherInFlight, ++step) {
    const int seg = __builtin_amdgcn_readfirstlane((int)((wave + step) % n_seg));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(table + (size_t)seg * seg_bytes, seg_bytes);
    i32x4 v[kGatherInFlight];
#pragma unroll
    for (int j = 0; j < kGatherInFlight; ++j) {
      const int64_t r = base + (int64_t)j * groups;
      const uint32_t off = r < n ? (uint32_t)rows[r] * 256u + 16u * s : 0x80000000u;
      v[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, AUX));
    }
#pragma unroll
    for (int j = 0; j < kGatherInFlight; ++j) x ^= (uint32_t)(v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3]);
  }
  block_xor_store(x, out);
}

// Read-only stream: 16-byte buffer loads, four in flight per lane; one load instruction of a
// wave reads 1 KiB contiguous, and thread t reads pieces t, t + S, ... (S threads in the
// grid).  The region goes in segments of at most 1 GiB, each behind its own buffer resource
// (32-bit offsets).  Global loads of the same pattern measured 5.0-5.6 TB/s against 6.1-6.6
// for these.  AUX: the loads' cache-policy operand (non-temporal for the ceiling; ordinary
// loads, which fill the caches, to evict other data from them).
constexpr int kReadInFlight = 4;
constexpr int64_t kReadSegment = (int64_t)1 << 30;

template <int AUX>
__global__ __launch_bounds__(kPeakBlock) void peak_read_kernel(const unsigned char* __restrict__ src,
                                                               int64_t bytes,
                                                               uint32_t* __restrict__ out) {
  const int64_t S = (int64_t)gridDim.x * kPeakBlock;
  const int64_t t = (int64_t)blockIdx.x * kPeakBlock + threadIdx.x;
  uint32_t x = 0;
  for (int64_t seg = 0; seg < bytes; seg += kReadSegment) {
    const int64_t sb = bytes - seg < kReadSegment ? bytes - seg : kReadSegment;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + seg, (uint32_t)sb);
    const int64_t n16 = sb / 16;
    for (int64_t i = t; i < n16; i += S * kReadInFlight) {
      i32x4 v[kReadInFlight];
#pragma unroll
      for (int j = 0; j < kReadInFlight; ++j) {
        const int64_t e = i + (int64_t)j * S;
        const uint32_t off = e < n16 ? (uint32_t)(e * 16) : 0x80000000u;
        v[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, AUX));
      }
#pragma unroll
      for (int j = 0; j < kReadInFlight; ++j) x ^= (uint32_t)(v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3]);
    }
  }
  block_xor_store(x, out);
}

struct SelArgs {
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* idx;
  const int32_t* kv_len;
  uint32_t* out;
  int B, T, S_max, H_kv, k, chunks, splits, chunks_per_split;
};

// The K and V rows of a selection, gathered as the sparse attention gathers them (one block
// per (query, KV head, split), wave w taking chunks w, w + 4, ... of 32 entries, 16-byte
// loads by D/8 consecutive lanes per row, the next two chunks in flight, XCD-aware block
// numbering) and XORed into a checksum instead of computed with.  Entries < 0 or past
// kv_len read nothing (buffer bounds), as in the attention.
template <int D>
__global__ __launch_bounds__(kPeakBlock) void peak_gather_selection_kernel(SelArgs p) {
  constexpr int ROWB = D * 2, PI = ROWB / 16, RPI = 64 / PI, NI = 32 / RPI, W = 4;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned bid = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
  const int split = bid % p.splits;
  const int64_t rk = bid / p.splits;
  const int kvh = (int)(rk % p.H_kv);
  const int64_t row = rk / p.H_kv;
  const int b = (int)(row / p.T);
  int kvl = p.kv_len ? p.kv_len[b] : p.S_max;
  kvl = __builtin_amdgcn_readfirstlane(kvl < 0 ? 0 : (kvl > p.S_max ? p.S_max : kvl));
  const int32_t* irow = p.idx + (size_t)row * p.k;
  const uint32_t stride_b = (uint32_t)(p.H_kv * ROWB);
  const size_t seq_off = ((size_t)b * p.S_max * p.H_kv + kvh) * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.kc + seq_off, (uint32_t)kvl * stride_b);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.vc + seq_off, (uint32_t)kvl * stride_b);
  const int rho = lane / PI, s = lane % PI;
  const int c_begin = split * p.chunks_per_split;
  const int c_end = min(c_begin + p.chunks_per_split, p.chunks);
  // as the attention: lane e_lane holds entry e_lane of a chunk as stored; the rows of slots
  // rho * NI + i are fetched with the keys taken from those lanes
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(irow, (uint32_t)p.k * 4u);
  const int e_lane = lane & 31;
  auto raw_of = [&](int c) -> int {
    const uint32_t off = c < c_end ? (uint32_t)(c * 32 + e_lane) * 4u : 0x80000000u;
    return __builtin_amdgcn_raw_buffer_load_b32(irs, (int)off, 0, 0);
  };
  auto issue = [&](int c, int j, i32x4 (&kd)[NI], i32x4 (&vd)[NI]) {
    const int e = c * 32 + e_lane;
    const int key = (c < c_end && e < p.k && j >= 0 && j < kvl) ? j : -1;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int jv = __shfl(key, rho * NI + i);
      const uint32_t off = jv >= 0 ? (uint32_t)jv * stride_b + 16u * s : 0x80000000u;
      kd[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
      vd[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, 0));
    }
  };
  uint32_t x = 0;
  auto consume = [&](const i32x4 (&kd)[NI], const i32x4 (&vd)[NI]) {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      x ^= (uint32_t)(kd[j][0] ^ kd[j][1] ^ kd[j][2] ^ kd[j][3] ^ vd[j][0] ^ vd[j][1] ^ vd[j][2] ^
                      vd[j][3]);
  };
  // as the attention: two register sets, each with the raw entries of its next chunk loaded
  // right after its rows, so two chunks' gathers are in flight while one is consumed
  i32x4 kA[NI], vA[NI], kB[NI], vB[NI];
  const int c0 = c_begin + wid;
  int jA = raw_of(c0), jB = raw_of(c0 + W);
  issue(c0, jA, kA, vA);
  jA = raw_of(c0 + 2 * W);
  issue(c0 + W, jB, kB, vB);
  jB = raw_of(c0 + 3 * W);
  auto step = [&](int c, i32x4 (&kd)[NI], i32x4 (&vd)[NI], int& jr) __attribute__((always_inline)) {
    consume(kd, vd);
    issue(c + 2 * W, jr, kd, vd);
    jr = raw_of(c + 4 * W);
  };
  int c = c0;
  for (; c + W < c_end; c += 2 * W) {
    step(c, kA, vA, jA);
    step(c + W, kB, vB, jB);
  }
  if (c < c_end) step(c, kA, vA, jA);
  block_xor_store(x, p.out);
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

}  // namespace ix

namespace {

thread_local std::string g_peak_err;

ix_status peak_fail(ix_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ix_status peak_fail(ix_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_peak_err = buf;
  return st;
}

ix_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return peak_fail(IX_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  g_peak_err.clear();
  return IX_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

const char* ix_peak_last_error(void) { return g_peak_err.c_str(); }

ix_status ix_peak_mfma_fp8(const void* operands, int32_t valu_per_mfma, int32_t blocks,
                           int32_t iters, float* out, hipStream_t stream) {
  using namespace ix;
  if (!operands || !out) return peak_fail(IX_ERR_INVALID, "NULL operands or out");
  if (blocks < 1 || iters < 1)
    return peak_fail(IX_ERR_INVALID, "blocks=%d iters=%d must be >= 1", blocks, iters);
  if (valu_per_mfma != 0 && valu_per_mfma != 4 && valu_per_mfma != 8 && valu_per_mfma != 12)
    return peak_fail(IX_ERR_INVALID, "valu_per_mfma=%d (0, 4, 8 or 12)", valu_per_mfma);
  if (!aligned16(operands)) return peak_fail(IX_ERR_INVALID, "operands must be 16-byte aligned");
  const i32x8* tab = reinterpret_cast<const i32x8*>(operands);
  const dim3 g((unsigned)blocks), b(kPeakBlock);
  switch (valu_per_mfma) {
    case 0: hipLaunchKernelGGL(peak_mfma_kernel<0>, g, b, 0, stream, tab, iters, out); break;
    case 4: hipLaunchKernelGGL(peak_mfma_kernel<4>, g, b, 0, stream, tab, iters, out); break;
    case 8: hipLaunchKernelGGL(peak_mfma_kernel<8>, g, b, 0, stream, tab, iters, out); break;
    default: hipLaunchKernelGGL(peak_mfma_kernel<12>, g, b, 0, stream, tab, iters, out); break;
  }
  return launched("ix_peak_mfma_fp8");
}

ix_status ix_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  using namespace ix;
  if (!src || !dst) return peak_fail(IX_ERR_INVALID, "NULL src or dst");
  if (bytes % 16 || !aligned16(src) || !aligned16(dst))
    return peak_fail(IX_ERR_INVALID, "bytes and both pointers must be multiples of 16");
  if (bytes == 0) return IX_OK;
  hipLaunchKernelGGL(peak_copy_kernel, dim3(kReadBlocks), dim3(kPeakBlock), 0, stream,
                     reinterpret_cast<const i32x4*>(src), reinterpret_cast<i32x4*>(dst),
                     (int64_t)(bytes / 16));
  return launched("ix_peak_copy");
}

ix_status ix_peak_read(const void* src, size_t bytes, int32_t blocks, int32_t nontemporal,
                       uint32_t* out, hipStream_t stream) {
  using namespace ix;
  if (!src || !out) return peak_fail(IX_ERR_INVALID, "NULL src or out");
  if (bytes % 16 || !aligned16(src))
    return peak_fail(IX_ERR_INVALID, "bytes and src must be multiples of 16");
  if (blocks < 1 || blocks > kMaxPeakBlocks)
    return peak_fail(IX_ERR_INVALID, "blocks=%d (1..%d)", blocks, kMaxPeakBlocks);
  if (nontemporal != 0 && nontemporal != 1)
    return peak_fail(IX_ERR_INVALID, "nontemporal=%d (0 or 1)", nontemporal);
  if (bytes == 0) return IX_OK;
  const unsigned char* s = reinterpret_cast<const unsigned char*>(src);
  if (nontemporal)
    hipLaunchKernelGGL(peak_read_kernel<kLoadNT>, dim3(blocks), dim3(kPeakBlock), 0, stream, s,
                       (int64_t)bytes, out);
  else
    hipLaunchKernelGGL(peak_read_kernel<0>, dim3(blocks), dim3(kPeakBlock), 0, stream, s,
                       (int64_t)bytes, out);
  return launched("ix_peak_read");
}

ix_status ix_peak_gather(const void* table, size_t table_bytes, const int32_t* rows, int64_t n,
                         int32_t blocks, uint32_t* out, hipStream_t stream) {
  using namespace ix;
  if (!table || !rows || !out) return peak_fail(IX_ERR_INVALID, "NULL table, rows or out");
  if (n < 0) return peak_fail(IX_ERR_INVALID, "n=%lld must be >= 0", (long long)n);
  if (blocks < 1 || blocks > kMaxPeakBlocks)
    return peak_fail(IX_ERR_INVALID, "blocks=%d (1..%d)", blocks, kMaxPeakBlocks);
  if (table_bytes == 0 || table_bytes % 256 || table_bytes > ((size_t)1 << 31))
    return peak_fail(IX_ERR_INVALID, "table_bytes must be a positive multiple of 256, at most 2 GiB");
  if (!aligned16(table)) return peak_fail(IX_ERR_INVALID, "table must be 16-byte aligned");
  if (n == 0) return IX_OK;
  hipLaunchKernelGGL(peak_gather_kernel<0>, dim3(blocks), dim3(kPeakBlock), 0, stream,
                     reinterpret_cast<const unsigned char*>(table), (uint32_t)table_bytes, 1, rows,
                     n, out);
  return launched("ix_peak_gather");
}

ix_status ix_peak_gather_wide(const void* table, size_t seg_bytes, int32_t n_seg,
                              const int32_t* rows, int64_t n, int32_t blocks, int32_t nontemporal,
                              uint32_t* out, hipStream_t stream) {
  using namespace ix;
  if (!table || !rows || !out) return peak_fail(IX_ERR_INVALID, "NULL table, rows or out");
  if (n < 0) return peak_fail(IX_ERR_INVALID, "n=%lld must be >= 0", (long long)n);
  if (blocks < 1 || blocks > kMaxPeakBlocks)
    return peak_fail(IX_ERR_INVALID, "blocks=%d (1..%d)", blocks, kMaxPeakBlocks);
  if (seg_bytes == 0 || seg_bytes % 256 || seg_bytes > ((size_t)1 << 30))
    return peak_fail(IX_ERR_INVALID, "seg_bytes must be a positive multiple of 256, at most 1 GiB");
  if (n_seg < 1 || n_seg > 64) return peak_fail(IX_ERR_INVALID, "n_seg=%d (1..64)", n_seg);
  if (nontemporal != 0 && nontemporal != 1)
    return peak_fail(IX_ERR_INVALID, "nontemporal=%d (0 or 1)", nontemporal);
  if (!aligned16(table)) return peak_fail(IX_ERR_INVALID, "table must be 16-byte aligned");
  if (n == 0) return IX_OK;
  auto kern = nontemporal ? peak_gather_kernel<kLoadNT> : peak_gather_kernel<0>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kPeakBlock), 0, stream,
                     reinterpret_cast<const unsigned char*>(table), (uint32_t)seg_bytes, (int)n_seg,
                     rows, n, out);
  return launched("ix_peak_gather_wide");
}

ix_status ix_peak_gather_selection(const void* kc, const void* vc, const int32_t* idx,
                                   const int32_t* kv_len, int32_t B, int32_t T, int32_t S_max,
                                   int32_t H_kv, int32_t d, int32_t k, int32_t splits,
                                   int32_t blocks_per_cu, uint32_t* out, hipStream_t stream) {
  using namespace ix;
  if (!kc || !vc || !idx || !out) return peak_fail(IX_ERR_INVALID, "NULL kc, vc, idx or out");
  if (B < 0 || T < 0 || S_max < 1 || H_kv < 1 || k < 1 || k > 2048 || splits < 1)
    return peak_fail(IX_ERR_INVALID, "sizes out of range (B=%d T=%d S_max=%d H_kv=%d k=%d splits=%d)",
                     B, T, S_max, H_kv, k, splits);
  if (d != 64 && d != 128) return peak_fail(IX_ERR_UNSUPPORTED, "d=%d unsupported (64 or 128)", d);
  if (blocks_per_cu != 0 && blocks_per_cu != 2 && blocks_per_cu != 3)
    return peak_fail(IX_ERR_INVALID, "blocks_per_cu=%d (0, 2 or 3)", blocks_per_cu);
  if (!aligned16(kc) || !aligned16(vc)) return peak_fail(IX_ERR_INVALID, "kc/vc must be 16-byte aligned");
  if ((int64_t)S_max * H_kv * d * 2 > ((int64_t)1 << 31))
    return peak_fail(IX_ERR_UNSUPPORTED, "one sequence's K (or V) cache must stay within 2 GiB");
  const int64_t blocks = (int64_t)B * T * H_kv * splits;
  if (blocks > (int64_t)0xFFFFFFFF / kPeakBlock)
    return peak_fail(IX_ERR_UNSUPPORTED, "%lld blocks: too many for one launch", (long long)blocks);
  if (blocks == 0) return IX_OK;
  SelArgs x{};
  x.kc = reinterpret_cast<const uint16_t*>(kc);
  x.vc = reinterpret_cast<const uint16_t*>(vc);
  x.idx = idx;
  x.kv_len = kv_len;
  x.out = out;
  x.B = B;
  x.T = T;
  x.S_max = S_max;
  x.H_kv = H_kv;
  x.k = k;
  x.chunks = (k + 31) / 32;
  x.splits = splits;
  x.chunks_per_split = (x.chunks + splits - 1) / splits;
  // an occupancy limit through unused dynamic LDS: 160 KiB per CU hold 2 blocks of 54 KiB,
  // 3 of 41 KiB
  const size_t lds = blocks_per_cu == 2 ? 54 * 1024 : blocks_per_cu == 3 ? 41 * 1024 : 0;
  if (d == 128)
    hipLaunchKernelGGL(peak_gather_selection_kernel<128>, dim3((unsigned)blocks), dim3(kPeakBlock),
                       lds, stream, x);
  else
    hipLaunchKernelGGL(peak_gather_selection_kernel<64>, dim3((unsigned)blocks), dim3(kPeakBlock),
                       lds, stream, x);
  return launched("ix_peak_gather_selection");
}

ix_status ix_peak_atomic_add(float* table, int64_t rows, const int32_t* idx, int64_t n,
                             hipStream_t stream) {
  using namespace ix;
  if (!table || !idx) return peak_fail(IX_ERR_INVALID, "NULL table or idx");
  if (rows < 1 || rows > ((int64_t)1 << 31) / 128 || n < 0)
    return peak_fail(IX_ERR_INVALID, "rows=%lld n=%lld out of range", (long long)rows, (long long)n);
  if (n == 0) return IX_OK;
  hipLaunchKernelGGL(peak_atomic_kernel, dim3(256 * 8), dim3(kPeakBlock), 0, stream, table, rows,
                     idx, n);
  return launched("ix_peak_atomic_add");
}

}  // extern "C"
