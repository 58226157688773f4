// Atomic-free accumulation of per-pair gradient rows into per-key rows, for the two
// backward passes whose key gradients sum over every query that kept a key: the sparse
// attention's dK / dV and the indexer's dk_I.  The fp32 atomic units of the L2 take about
// one 32-bit add per clock per channel, which bounds the atomic form at one add per
// gradient element per kept pair.  Instead, per pass over a range of query rows:
//  1. count the kept pairs of each key (b, s) per block of consecutive query rows, scan the
//     keys' totals into segment offsets, and split each segment by row block: key g's
//     segment holds block 0's pairs, then block 1's, and so on;
//  2. list every pair's position in the pass under its key (the inverted selection): one
//     workgroup per row block takes its rows in order, so each key's pairs come in row
//     order and the lists, and the sums below, are the same on every run;
//  3. the gradient kernel writes each pair's rows (bf16, or fp32 at the caller's choice) in
//     pair order;
//  4. one wave per (key, head) sums its pairs' rows (each read once, non-temporal) in fp32
//     and adds the sums to the gradient rows with ordinary loads and stores (the wave owns
//     those rows).
// Only entries of one query row that repeat a key take an arrival order among themselves.
// The attention's rows of such entries are equal, so their order changes nothing there.
#include <algorithm>
#include <type_traits>

#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

constexpr int kScanThreads = 256;
constexpr int kScanPer = 8;
constexpr int kScanTile = kScanThreads * kScanPer;
constexpr int kPairUnroll = 16;  // pair rows in flight per wave in the key sums
constexpr int64_t kMaxSlots = (int64_t)1 << 26;  // (key, row block) counters per pass
constexpr int64_t kBlkChunk = 64;                // row blocks per partial sum

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

__global__ __launch_bounds__(256) void pair_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// Key id b * S_max + s of pair e of the pass (query row row0 + e / k, entry e % k), or -1
// for padding (s < 0 or s >= kv_len[b], kv_len clamped to S_max; NULL kv_len: S_max).
__device__ __forceinline__ int64_t pair_key(const int32_t* idx, const int32_t* kv_len, int T,
                                            int S_max, int k, int64_t row0, int64_t e) {
  const int64_t row = row0 + e / k;
  const int b = (int)(row / T);
  int kvl = kv_len ? kv_len[b] : S_max;
  kvl = kvl < 0 ? 0 : (kvl > S_max ? S_max : kvl);
  const int s = idx[row * k + e % k];
  return (s >= 0 && s < kvl) ? (int64_t)b * S_max + s : -1;
}

// Counts per (row block, key), block-major: cnt[((row in pass) / rows_per_blk) * n_keys + g].
__global__ __launch_bounds__(256) void pair_count_kernel(const int32_t* idx, const int32_t* kv_len,
                                                         int T, int S_max, int k, int64_t row0,
                                                         int64_t pairs, int64_t n_keys,
                                                         int64_t rows_per_blk, uint32_t* cnt) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < pairs; e += (int64_t)gridDim.x * 256) {
    const int64_t g = pair_key(idx, kv_len, T, S_max, k, row0, e);
    if (g >= 0) atomicAdd(cnt + ((e / k) / rows_per_blk) * n_keys + g, 1u);
  }
}

// Row blocks are taken in chunks of kBlkChunk.  part_sum[c * n_keys + g] = key g's pairs in
// chunk c of the row blocks.
__global__ __launch_bounds__(256) void pair_chunk_sums(const uint32_t* cnt, int64_t n_keys,
                                                       int64_t n_blk, uint32_t* part_sum) {
  const int64_t n_chunks = (n_blk + kBlkChunk - 1) / kBlkChunk;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < n_chunks * n_keys;
       it += (int64_t)gridDim.x * 256) {
    const int64_t c = it / n_keys, g = it % n_keys;
    const int64_t b1 = std::min<int64_t>(n_blk, (c + 1) * kBlkChunk);
    uint32_t t = 0;
    for (int64_t blk = c * kBlkChunk; blk < b1; ++blk) t += cnt[blk * n_keys + g];
    part_sum[it] = t;
  }
}

// tot[g] = key g's pairs over all row blocks (tot[n_keys] = 0, the scan's end slot).
__global__ __launch_bounds__(256) void pair_key_totals(const uint32_t* part_sum, int64_t n_keys,
                                                       int64_t n_chunks, uint32_t* tot) {
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g <= n_keys; g += (int64_t)gridDim.x * 256) {
    uint32_t t = 0;
    if (g < n_keys)
      for (int64_t c = 0; c < n_chunks; ++c) t += part_sum[c * n_keys + g];
    tot[g] = t;
  }
}

// With tot scanned into segment offsets: cnt[blk][g] becomes where row block blk's pairs of
// key g start (the segment start plus the earlier blocks' counts).
__global__ __launch_bounds__(256) void pair_block_offsets(uint32_t* cnt, int64_t n_keys,
                                                          int64_t n_blk, const uint32_t* part_sum,
                                                          const uint32_t* off) {
  const int64_t n_chunks = (n_blk + kBlkChunk - 1) / kBlkChunk;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < n_chunks * n_keys;
       it += (int64_t)gridDim.x * 256) {
    const int64_t c = it / n_keys, g = it % n_keys;
    uint32_t run = off[g];
    for (int64_t c2 = 0; c2 < c; ++c2) run += part_sum[c2 * n_keys + g];
    const int64_t b1 = std::min<int64_t>(n_blk, (c + 1) * kBlkChunk);
    for (int64_t blk = c * kBlkChunk; blk < b1; ++blk) {
      const uint32_t v = cnt[blk * n_keys + g];
      cnt[blk * n_keys + g] = run;
      run += v;
    }
  }
}

// Block-wide exclusive scan of one value per thread; the block total goes to *total.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  uint32_t base = 0, all = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wid) base += wsum[w];
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return base + x - v;
}

__global__ __launch_bounds__(kScanThreads) void pair_scan_tiles(const uint32_t* cnt, int64_t n,
                                                               uint32_t* part) {
  __shared__ uint32_t wsum[kScanThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanPer;
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i)
    if (base + i < n) v += cnt[base + i];
  uint32_t total;
  block_exclusive_scan(v, wsum, &total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// One block: exclusive scan of the tile totals, in place.
__global__ __launch_bounds__(1024) void pair_scan_top(uint32_t* part, int64_t nparts) {
  __shared__ uint32_t wsum[16];
  uint32_t carry = 0;
  for (int64_t i0 = 0; i0 < nparts; i0 += 1024) {
    const int64_t i = i0 + threadIdx.x;
    const uint32_t v = i < nparts ? part[i] : 0u;
    uint32_t total;
    const uint32_t ex = block_exclusive_scan(v, wsum, &total);
    if (i < nparts) part[i] = carry + ex;
    carry += total;
  }
}

__global__ __launch_bounds__(kScanThreads) void pair_scan_apply(uint32_t* cnt, int64_t n,
                                                               const uint32_t* part) {
  __shared__ uint32_t wsum[kScanThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanPer;
  uint32_t v[kScanPer], sum = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    v[i] = base + i < n ? cnt[base + i] : 0u;
    sum += v[i];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan(sum, wsum, &total) + part[blockIdx.x];
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    if (base + i < n) cnt[base + i] = run;
    run += v[i];
  }
}

// One workgroup per row block, its rows one at a time: the entries of a row are spread over
// the threads, and a barrier separates rows, so a slot's cursor counts the block's earlier
// rows and each key lists its pairs in row order.
__global__ __launch_bounds__(256) void pair_fill_inv_kernel(const int32_t* idx, const int32_t* kv_len,
                                                            int T, int S_max, int k, int64_t row0,
                                                            int64_t rows, int64_t n_keys,
                                                            int64_t rows_per_blk,
                                                            const uint32_t* start, uint32_t* cur,
                                                            uint32_t* inv) {
  constexpr int kPer = 8;  // entries of a row per thread, all in flight together
  const int64_t blk = blockIdx.x;
  const uint32_t* st = start + blk * n_keys;
  uint32_t* cu = cur + blk * n_keys;
  const int64_t r_end = std::min<int64_t>(rows, (blk + 1) * rows_per_blk);
  for (int64_t r = blk * rows_per_blk; r < r_end; ++r) {
    for (int j0 = 0; j0 < k; j0 += 256 * kPer) {
      int64_t g[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int j = j0 + i * 256 + (int)threadIdx.x;
        g[i] = j < k ? pair_key(idx, kv_len, T, S_max, k, row0, r * k + j) : -1;
      }
      uint32_t pos[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) pos[i] = g[i] >= 0 ? st[g[i]] + atomicAdd(cu + g[i], 1u) : 0u;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (g[i] >= 0) inv[pos[i]] = (uint32_t)(r * k + j0 + i * 256 + (int)threadIdx.x);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v) {
  return __builtin_bit_cast(float, v << 16);
}

// One wave per (key, head), grid-stride over all of them.  Key g's pairs are
// inv[off[g] .. off[g + 1]).  A pair's row for head h is W elements (bf16, or fp32 with F32)
// at contrib + (pair * H + h) * W; lanes 0..31 sum elements [0, W/2) into dst_a, lanes 32..63
// elements [W/2, W) into dst_b, EPL consecutive columns each; the sums are added to row
// (key * H + h) of stride `stride` floats.
template <int W, bool F32>
__global__ __launch_bounds__(256) void pair_reduce_kernel(const uint32_t* off, const uint32_t* inv,
                                                          const void* contrib, int64_t n_keys,
                                                          int H, float* dst_a, float* dst_b,
                                                          int64_t stride) {
  constexpr int EPL = W / kWave;
  static_assert(EPL == 1 || EPL == 2 || EPL == 4, "row width");
  const int lane = threadIdx.x & 63;
  const int part = lane >> 5;
  const int col = (lane & 31) * EPL;
  const int64_t waves = ((int64_t)gridDim.x * 256) >> 6;
  using Elem = std::conditional_t<F32, float, uint16_t>;
  const Elem* rows_base = reinterpret_cast<const Elem*>(contrib);
  for (int64_t it = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6; it < n_keys * H; it += waves) {
    const int64_t g = it / H;
    const int h = (int)(it % H);
    const uint32_t n0 = off[g], n1 = off[g + 1];
    if (n0 == n1) continue;
    float acc[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
    // this lane's EPL elements of one pair row, and their sum into acc
    using Raw = std::conditional_t<
        F32, std::conditional_t<EPL == 4, float4, std::conditional_t<EPL == 2, float2, float>>,
        std::conditional_t<EPL == 4, uint2, std::conditional_t<EPL == 2, uint32_t, uint16_t>>>;
    // each pair row is read once: non-temporal loads (as ext-vector words of the same size)
    auto load_pair = [&](uint32_t pr) -> Raw {
      const void* ptr = rows_base + ((size_t)pr * H + h) * W + part * (W / 2) + col;
      typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
      typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
      if constexpr (sizeof(Raw) == 16) {
        return __builtin_bit_cast(Raw, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(ptr)));
      } else if constexpr (sizeof(Raw) == 8) {
        return __builtin_bit_cast(Raw, __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(ptr)));
      } else if constexpr (sizeof(Raw) == 4) {
        return __builtin_bit_cast(Raw, __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ptr)));
      } else {
        return __builtin_bit_cast(Raw, __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(ptr)));
      }
    };
    auto add_raw = [&](Raw v) {
      if constexpr (F32) {
        if constexpr (EPL == 4) {
          acc[0] += v.x;
          acc[1] += v.y;
          acc[2] += v.z;
          acc[3] += v.w;
        } else if constexpr (EPL == 2) {
          acc[0] += v.x;
          acc[1] += v.y;
        } else {
          acc[0] += v;
        }
      } else if constexpr (EPL == 4) {
        acc[0] += bf16_bits_to_f32(v.x & 0xFFFFu);
        acc[1] += bf16_bits_to_f32(v.x >> 16);
        acc[2] += bf16_bits_to_f32(v.y & 0xFFFFu);
        acc[3] += bf16_bits_to_f32(v.y >> 16);
      } else if constexpr (EPL == 2) {
        acc[0] += bf16_bits_to_f32(v & 0xFFFFu);
        acc[1] += bf16_bits_to_f32(v >> 16);
      } else {
        acc[0] += bf16_bits_to_f32(v);
      }
    };
    // The key's pair rows, kPairUnroll at a time, summed in segment order: the rows of a
    // group are all in flight at once, and the positions of the next group load meanwhile.
    constexpr int U = kPairUnroll;
    uint32_t e = n0;
    if (n1 - n0 >= (uint32_t)U) {
      uint32_t pr[U];
#pragma unroll
      for (int i = 0; i < U; ++i) pr[i] = inv[e + i];
      while (true) {
        const uint32_t en = e + U;
        const bool more = en + U <= n1;
        uint32_t nx[U] = {};
        if (more) {
#pragma unroll
          for (int i = 0; i < U; ++i) nx[i] = inv[en + i];
        }
        Raw raw[U];
#pragma unroll
        for (int i = 0; i < U; ++i) raw[i] = load_pair(pr[i]);
#pragma unroll
        for (int i = 0; i < U; ++i) add_raw(raw[i]);
        e = en;
        if (!more) break;
#pragma unroll
        for (int i = 0; i < U; ++i) pr[i] = nx[i];
      }
    }
    for (; e < n1; ++e) add_raw(load_pair(inv[e]));
    float* dst = (part ? dst_b : dst_a) + ((size_t)g * H + h) * stride + col;
#pragma unroll
    for (int i = 0; i < EPL; ++i) dst[i] += acc[i];
  }
}

dim3 grid_for(int64_t n) { return dim3((unsigned)std::min<int64_t>((n + 255) / 256, 65536)); }

}  // namespace

PairLayout pair_layout(int B, int S_max, int k, int64_t rows, size_t row_bytes) {
  PairLayout L{};
  L.n_keys = (int64_t)B * S_max;
  // row blocks: at least 8 rows each, and at most 2^26 (key, block) slots in all
  const int64_t by_slots = std::max<int64_t>(1, kMaxSlots / std::max<int64_t>(L.n_keys, 1));
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>((rows + 7) / 8, by_slots));
  L.rows_per_blk = std::max<int64_t>(1, (rows + want - 1) / want);
  L.n_blk = std::max<int64_t>(1, (rows + L.rows_per_blk - 1) / L.rows_per_blk);
  L.n_slots = L.n_keys * L.n_blk;
  L.nparts = (L.n_keys + 1 + kScanTile - 1) / kScanTile;
  L.off = 0;
  L.cnt = L.off + up256((size_t)(L.n_keys + 1) * 4);
  L.cur = L.cnt + up256((size_t)L.n_slots * 4);
  L.part_sum = L.cur + up256((size_t)L.n_slots * 4);
  L.part = L.part_sum + up256((size_t)((L.n_blk + kBlkChunk - 1) / kBlkChunk) * L.n_keys * 4);
  L.inv = L.part + up256((size_t)L.nparts * 4);
  L.contrib = L.inv + up256((size_t)rows * k * 4);
  L.total = L.contrib + up256((size_t)rows * k * row_bytes);
  return L;
}

int64_t pair_rows_per_pass(int B, int T, int S_max, int k, size_t row_bytes, size_t ws_bytes) {
  const int64_t all = (int64_t)B * T;
  // pair positions are 32-bit: at most 2^31 pairs per pass
  int64_t hi = std::min<int64_t>(all, ((int64_t)1 << 31) / k);
  if (pair_layout(B, S_max, k, 1, row_bytes).total > ws_bytes) return 0;
  int64_t lo = 1;
  while (lo < hi) {  // the largest row count that fits
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (pair_layout(B, S_max, k, mid, row_bytes).total <= ws_bytes) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

hipError_t launch_pair_index(const int32_t* idx, const int32_t* kv_len, int T, int S_max, int k,
                             int64_t row0, int64_t rows, const PairLayout& L, void* ws,
                             hipStream_t stream) {
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* off = reinterpret_cast<uint32_t*>(w + L.off);
  uint32_t* cur = reinterpret_cast<uint32_t*>(w + L.cur);
  uint32_t* part = reinterpret_cast<uint32_t*>(w + L.part);
  uint32_t* inv = reinterpret_cast<uint32_t*>(w + L.inv);
  const int64_t pairs = rows * k;
  uint32_t* cnt = reinterpret_cast<uint32_t*>(w + L.cnt);
  hipLaunchKernelGGL(pair_zero_kernel, grid_for(L.n_slots), dim3(256), 0, stream, cnt, L.n_slots);
  hipLaunchKernelGGL(pair_zero_kernel, grid_for(L.n_slots), dim3(256), 0, stream, cur, L.n_slots);
  hipLaunchKernelGGL(pair_count_kernel, grid_for(pairs), dim3(256), 0, stream, idx, kv_len, T, S_max,
                     k, row0, pairs, L.n_keys, L.rows_per_blk, cnt);
  uint32_t* part_sum = reinterpret_cast<uint32_t*>(w + L.part_sum);
  const int64_t n_chunks = (L.n_blk + kBlkChunk - 1) / kBlkChunk;
  hipLaunchKernelGGL(pair_chunk_sums, grid_for(n_chunks * L.n_keys), dim3(256), 0, stream, cnt,
                     L.n_keys, L.n_blk, part_sum);
  hipLaunchKernelGGL(pair_key_totals, grid_for(L.n_keys + 1), dim3(256), 0, stream, part_sum,
                     L.n_keys, n_chunks, off);
  hipLaunchKernelGGL(pair_scan_tiles, dim3((unsigned)L.nparts), dim3(kScanThreads), 0, stream, off,
                     L.n_keys + 1, part);
  hipLaunchKernelGGL(pair_scan_top, dim3(1), dim3(1024), 0, stream, part, L.nparts);
  hipLaunchKernelGGL(pair_scan_apply, dim3((unsigned)L.nparts), dim3(kScanThreads), 0, stream, off,
                     L.n_keys + 1, part);
  hipLaunchKernelGGL(pair_block_offsets, grid_for(n_chunks * L.n_keys), dim3(256), 0, stream, cnt,
                     L.n_keys, L.n_blk, part_sum, off);
  hipLaunchKernelGGL(pair_fill_inv_kernel, dim3((unsigned)L.n_blk), dim3(256), 0, stream, idx, kv_len,
                     T, S_max, k, row0, rows, L.n_keys, L.rows_per_blk, cnt, cur, inv);
  return hipGetLastError();
}

hipError_t launch_pair_reduce(const PairLayout& L, const void* ws, int row_width, bool f32_rows,
                              int H, float* dst_a, float* dst_b, int64_t stride,
                              hipStream_t stream) {
  const char* w = reinterpret_cast<const char*>(ws);
  const uint32_t* off = reinterpret_cast<const uint32_t*>(w + L.off);
  const uint32_t* inv = reinterpret_cast<const uint32_t*>(w + L.inv);
  const void* contrib = w + L.contrib;
  const int64_t items = L.n_keys * H;
  const dim3 grid((unsigned)std::min<int64_t>((items + 3) / 4, 65536));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, off, inv, contrib, L.n_keys, H, dst_a,
                       dst_b, stride);
  };
  switch (row_width) {
    case 256: f32_rows ? go(pair_reduce_kernel<256, true>) : go(pair_reduce_kernel<256, false>); break;
    case 128: f32_rows ? go(pair_reduce_kernel<128, true>) : go(pair_reduce_kernel<128, false>); break;
    case 64: f32_rows ? go(pair_reduce_kernel<64, true>) : go(pair_reduce_kernel<64, false>); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ix
