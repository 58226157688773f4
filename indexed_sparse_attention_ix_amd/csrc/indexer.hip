// FP8 indexer (Stage 1, coarse scoring) fused with the streaming top-k (Stage 2, fine
// selection) of "DeepSeek Sparse Attention" as described in "GLM 5.2: How Four
// Co-Designed Mechanisms Beat Raw Scale", Part II.  Indexer form:
//   score(t,s) = sum_h w[t,h] * max(0, q_I[t,h,:] . k_I[s,:])
//
// Work unit: one wavefront owns QC query tokens of one sequence and one key split.
// Its queries' FP8 rows stay in VGPRs as MFMA B operands for the whole key sweep;
// key tiles of 16 rows stream from HBM/L2 straight into VGPRs as A operands
// (a ring of prefetched tiles), one 16x16x128 FP8 MFMA per (key tile, head block).
// The MFMA output columns are (query, head) pairs, so the ReLU + head-weight epilogue
// accumulates in-lane across head blocks and only HC adjacent lanes are summed at
// the end of a tile (DPP).  Tiles past the causal limit of the wave's last query are
// never visited.
//
// Selection keys are 64-bit: (order-preserving score bits << 32) | ~key_index, so
// larger key = better score, then lower index; all keys are distinct and the result
// does not depend on processing order.  Each (query, split) owns a candidate buffer
// in the workspace: keys >= the running threshold are appended in ascending key-index
// order; when a buffer nears capacity, a wave-level radix select over it finds a new
// threshold that keeps at least k entries and the buffer is compacted in place
// (order preserved).  At the end an exact select leaves exactly min(k, count)
// entries, already in ascending index order, so no sort is needed.
#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

constexpr int kBlockWaves = 4;
constexpr int kBlock = kBlockWaves * kWave;
constexpr int kHistBins = 256;
constexpr int kHistBatch = 4;  // 16-byte loads in flight per lane in a histogram pass

struct IxArgs {
  const uint8_t* q;
  const uint8_t* k;
  const float* w;
  const int32_t* q_pos0;
  const int32_t* kv_len;
  int B, T, S_max, H_I;
  int g;          // head blocks actually used (<= GMAX)
  int qgroups;    // query groups per sequence (over the row window for ix_score)
  int n_splits, split_len, cap, ksel;
  int64_t units;
  int t_begin, rows;  // ix_score row window
  uint64_t* cand;
  int32_t* cand_cnt;
  int32_t* idx;
  float* sel;
  float* scores;
};

// 32 bytes of an FP8 row for lane group lg (bytes [32*lg, 32*lg + 32)); rows of width
// 64 only fill lane groups 0 and 1, the other depth slots stay zero.
template <int DI>
__device__ __forceinline__ i32x8 load_row_slice(const uint8_t* row, int lg) {
  i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
  if (DI == 128 || lg < 2) {
    const i32x4 a = ld_global_16(row + 32 * lg);
    const i32x4 b = ld_global_16(row + 32 * lg + 16);
    v = (i32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return v;
}

__device__ __forceinline__ int visible_keys(int pos0, int kvl, int t) {
  const long v = (long)pos0 + t + 1;
  return (int)(v < 0 ? 0 : (v > kvl ? kvl : v));
}

// Per-wave query operands: B operands for every head block and the matching weights.
template <int QC, int GMAX, int DI>
struct QueryOperands {
  i32x8 bq[GMAX];
  float wv[GMAX];

  __device__ __forceinline__ void load(const IxArgs& p, int b, int t, bool valid, int safe_t,
                                       int j, int lg) {
    constexpr int HC = 16 / QC;
    const int tq = valid ? t : safe_t;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      bq[g] = (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
      wv[g] = 0.f;
      if (g < p.g) {
        const int head = g * HC + j;
        const size_t row = ((size_t)b * p.T + tq) * p.H_I + head;
        bq[g] = load_row_slice<DI>(p.q + row * DI, lg);
        wv[g] = valid ? p.w[row] : 0.f;
      }
    }
  }

  // ReLU on the float bits: a signed-integer max with 0 maps every negative float
  // (sign bit set) and -0 to +0 and leaves non-negative floats unchanged; one VALU op.
  static __device__ __forceinline__ float relu(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
  }
  static __device__ __forceinline__ void accumulate(f32x4& acc, const f32x4& x, float w) {
    acc[0] = fmaf(w, relu(x[0]), acc[0]);
    acc[1] = fmaf(w, relu(x[1]), acc[1]);
    acc[2] = fmaf(w, relu(x[2]), acc[2]);
    acc[3] = fmaf(w, relu(x[3]), acc[3]);
  }

  // Score of one (query, key) pair per lane for the 16-key tile held in `a`.
  // Lane l ends up with key 4*(l>>4) + (j & 3) and query (l & 15) / HC, where
  // j = (l & 15) % HC; for HC = 16 only lanes with j < 4 carry a distinct pair.
  // EXACT: all GMAX head blocks are used; the MFMA of block g+1 is issued before the
  // epilogue of block g so that the matrix core and the VALU overlap.
  template <bool EXACT>
  __device__ __forceinline__ float tile_score(const i32x8& a, int g_rt, int jsel) const {
    constexpr int HC = 16 / QC;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EXACT) {
      f32x4 x = mfma_e4m3_16x16x128(a, bq[0]);
#pragma unroll
      for (int g = 1; g < GMAX; ++g) {
        const f32x4 y = mfma_e4m3_16x16x128(a, bq[g]);
        accumulate(acc, x, wv[g - 1]);
        x = y;
      }
      accumulate(acc, x, wv[GMAX - 1]);

    } else {
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g < g_rt) accumulate(acc, mfma_e4m3_16x16x128(a, bq[g]), wv[g]);
      }
    }
    const bool b1 = (jsel & 2) != 0, b0 = (jsel & 1) != 0;
    const float keep0 = b1 ? acc[2] : acc[0], send0 = b1 ? acc[0] : acc[2];
    const float keep1 = b1 ? acc[3] : acc[1], send1 = b1 ? acc[1] : acc[3];
    const float c0 = keep0 + dpp_f32<kDppQuadXor2>(send0);
    const float c1 = keep1 + dpp_f32<kDppQuadXor2>(send1);
    float v = (b0 ? c1 : c0) + dpp_f32<kDppQuadXor1>(b0 ? c0 : c1);
    if (HC == 16) {
      v += dpp_f32<kDppRowRor4>(v);
      v += dpp_f32<kDppRowRor8>(v);
    }
    return v;
  }
};

// ------------------------------------------------------------------ wave-level select

struct SelectResult {
  uint64_t theta;  // keep entries >= theta
  int kept;        // how many entries that keeps
};

// Finds, within the 256 bins of `hist`, the digit holding the `needed`-th largest entry
// (counting from the top digit).  Returns digit, entries in higher digits, digit count.
__device__ __forceinline__ void wave_pick_digit(const uint32_t* hist, int nbins, uint32_t needed,
                                                int& digit, uint32_t& above, uint32_t& count) {
  const int lane = threadIdx.x & 63;
  uint32_t h[4];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bin = 4 * lane + i;
    h[i] = bin < nbins ? hist[bin] : 0u;
    s += h[i];
  }
  // suffix sum over lanes: sum of s over lanes >= lane
  uint32_t suf = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(suf, off);
    if (lane + off < 64) suf += o;
  }
  uint32_t a = suf - s;  // entries in lanes above this one
  int found = -1;
  uint32_t fa = 0, fh = 0;
#pragma unroll
  for (int i = 3; i >= 0; --i) {
    if (found < 0 && a < needed && needed <= a + h[i]) {
      found = 4 * lane + i;
      fa = a;
      fh = h[i];
    }
    a += h[i];
  }
  const uint64_t m = ballot64(found >= 0);
  const int src = __builtin_ctzll(m);
  digit = __shfl(found, src);
  above = __shfl(fa, src);
  count = __shfl(fh, src);
}

// 16-byte view of entries (e, e+1) of a candidate buffer.  Buffers start 16-byte aligned
// and have an even capacity, so for even e < n <= capacity the pair stays inside.
__device__ __forceinline__ void load_pair(const uint64_t* buf, int e, int n, uint64_t& x0,
                                          uint64_t& x1) {
  if (e < n) {
    const i32x4 v = ld_global_16(buf + e);
    x0 = ((uint64_t)(uint32_t)v[1] << 32) | (uint32_t)v[0];
    x1 = ((uint64_t)(uint32_t)v[3] << 32) | (uint32_t)v[2];
  } else {
    x0 = x1 = 0ull;
  }
}

// Histogram of the digit (v >> shift) & dmask over the entries of buf[0, n) whose bits
// at and above hs equal prefix.  Lane l reads entries 2l, 2l+1 of each 128-entry chunk;
// kHistBatch chunks are loaded before any is counted, so the L2 latency is paid once per
// 128 * kHistBatch entries.
__device__ void wave_hist(const uint64_t* buf, int n, uint64_t prefix, int hs, int shift,
                          uint32_t dmask, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  for (int e0 = 0; e0 < n; e0 += 128 * kHistBatch) {
    uint64_t x[kHistBatch][2];
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) load_pair(buf, e0 + 128 * u + 2 * lane, n, x[u][0], x[u][1]);
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = e0 + 128 * u + 2 * lane + j;
        const bool in = e < n && (hs >= 64 || (x[u][j] >> hs) == prefix);
        if (in) atomicAdd(&hist[(uint32_t)(x[u][j] >> shift) & dmask], 1u);
      }
    }
  }
}

// Radix select over buf[0, n) (distinct keys, all sharing their bits above `rem`
// equal to `prefix`).  Keeps the k largest: returns theta with #(v >= theta) = kept,
// where kept == k when exact, else the first kept <= limit reached while refining.
__device__ SelectResult wave_radix_select(const uint64_t* buf, int n, int k, int limit,
                                          uint64_t prefix, int rem, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t needed = (uint32_t)k;
  while (true) {
    const int dbits = rem < 8 ? rem : 8;
    const int shift = rem - dbits;
    const int nbins = 1 << dbits;
    for (int i = lane; i < kHistBins; i += 64) hist[i] = 0u;
    lds_wait();
    wave_hist(buf, n, prefix, rem, shift, (uint32_t)(nbins - 1), hist);
    lds_wait();
    int d;
    uint32_t above, cnt;
    wave_pick_digit(hist, nbins, needed, d, above, cnt);
    lds_wait();
    needed -= above;
    prefix = (prefix << dbits) | (uint64_t)d;
    rem = shift;
    const int kept = (int)(k - needed + cnt);
    if (cnt == needed || rem == 0 || kept <= limit) {
      return {rem >= 64 ? 0ull : (prefix << rem), kept};
    }
  }
}

// Common-prefix start for a select over keys whose high words lie in [mn_hi, mx_hi].
__device__ __forceinline__ void select_start(uint32_t mn_hi, uint32_t mx_hi, uint64_t& prefix,
                                             int& rem) {
  if (mn_hi == mx_hi) {
    prefix = mx_hi;
    rem = 32;
  } else {
    const uint32_t diff = mn_hi ^ mx_hi;
    const int hb = 31 - __builtin_clz(diff);  // highest differing bit of the high word
    rem = 32 + hb + 1;
    prefix = rem >= 64 ? 0ull : (((uint64_t)mx_hi << 32) >> rem);
  }
}

// Walks buf[0, n) in order and calls out(pos, v) for each entry >= theta, pos being its
// rank among the kept entries; returns how many were kept.  Lane l handles entries
// 2l, 2l+1 of each 128-entry chunk; four chunks are loaded before any is written, and
// a write never lands past the entry it came from, so in-place use is safe.
template <typename Out>
__device__ int wave_filter(const uint64_t* buf, int n, uint64_t theta, Out&& out) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lanemask_lt();
  int total = 0;
  for (int e0 = 0; e0 < n; e0 += 128 * 4) {
    uint64_t x[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) load_pair(buf, e0 + 128 * u + 2 * lane, n, x[u][0], x[u][1]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + 128 * u + 2 * lane;
      const bool k0 = e < n && x[u][0] >= theta;
      const bool k1 = e + 1 < n && x[u][1] >= theta;
      const uint64_t b0 = ballot64(k0), b1 = ballot64(k1);
      const int pos = total + popc64(b0 & lt) + popc64(b1 & lt);
      if (k0) out(pos, x[u][0]);
      if (k1) out(pos + (k0 ? 1 : 0), x[u][1]);
      total += popc64(b0) + popc64(b1);
    }
  }
  return total;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, (uint32_t)__shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ void mem_fence_wave() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
}

// One 16-row key tile as the A operand: lane (row r, group g) gets bytes [32g, 32g+32) of
// its row (rows of width 64 repeat bytes [32(g&1), ...) in groups 2, 3; the query
// operand is zero there, so they add nothing).
__device__ __forceinline__ i32x8 load_key_tile(__amdgpu_buffer_rsrc_t rs, int off) {
  const i32x4 lo = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  const i32x4 hi =
      __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
  return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ------------------------------------------------------------------ fused indexer + top-k

// Smallest and largest high word (score bits) over buf[0, n), wave-reduced.
__device__ void wave_hi_range(const uint64_t* buf, int n, uint32_t& mn, uint32_t& mx) {
  const int lane = threadIdx.x & 63;
  mn = 0xFFFFFFFFu;
  mx = 0u;
  for (int e0 = 0; e0 < n; e0 += 128 * kHistBatch) {
    uint64_t x[kHistBatch][2];
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) load_pair(buf, e0 + 128 * u + 2 * lane, n, x[u][0], x[u][1]);
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (e0 + 128 * u + 2 * lane + j < n) {
          mn = min(mn, (uint32_t)(x[u][j] >> 32));
          mx = max(mx, (uint32_t)(x[u][j] >> 32));
        }
      }
    }
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
}

// Low word of a selection key: ~s with bits 29-30 replaced by the query's slot in the
// wave (keys stay below 2^29, where those bits of ~s are always set), so one LDS stage
// can hold all of a wave's queries and ordering among one query's keys is unchanged.
constexpr uint32_t kTagShift = 29;
constexpr uint32_t kIndexMask = (1u << kTagShift) - 1u;
__device__ __forceinline__ uint32_t tagged_lo_base(int slot) {
  return 0x9FFFFFFFu | ((uint32_t)slot << kTagShift);  // minus s gives the tagged ~s
}
__device__ __forceinline__ int32_t untag_index(uint64_t key) {
  return (int32_t)(kIndexMask - ((uint32_t)key & kIndexMask));
}

template <int QC, int GMAX, int DI, bool EXACT>
__global__ __launch_bounds__(kBlock, 2) void ix_topk_partial_kernel(IxArgs p) {
  constexpr int HC = 16 / QC;
  // key tiles in flight per wave (the 16-block case keeps 128 VGPRs of query operands)
  constexpr int PF = GMAX >= 16 ? 2 : 4;
  constexpr int WSTG = 2 * 64 * PF;  // wave stage: two blocks of appends from every lane
  __shared__ uint32_t hist_all[kBlockWaves][kHistBins];
  __shared__ uint64_t stage_all[kBlockWaves][WSTG];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  uint32_t* hist = hist_all[wid];
  uint64_t* stage = stage_all[wid];
  const int64_t u = (int64_t)blockIdx.x * kBlockWaves + wid;
  if (u >= p.units) return;
  const int split = (int)(u % p.n_splits);
  const int64_t r = u / p.n_splits;
  const int b = (int)(r % p.B);
  const int qg = p.qgroups - 1 - (int)(r / p.B);  // latest (heaviest) query groups first
  const int t0 = qg * QC;
  const int r16 = lane & 15, lg = lane >> 4;
  const int qi = r16 / HC, j = r16 % HC;
  const int jsel = j & 3;
  const int t = t0 + qi;
  const bool qvalid = t < p.T;

  const int pos0 = p.q_pos0[b];
  int kvl = p.kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > p.S_max ? p.S_max : kvl);
  const int n_q = qvalid ? visible_keys(pos0, kvl, t) : 0;
  const int t_last = (t0 + QC < p.T ? t0 + QC : p.T) - 1;
  const int n_max = visible_keys(pos0, kvl, t_last);
  const int ks = split * p.split_len;
  const int ke = min(ks + p.split_len, n_max);

  QueryOperands<QC, GMAX, DI> qo;
  qo.load(p, b, t, qvalid, t0, j, lg);

  // lane constants: key offset of the lane's pair within a tile, the bound on candidate
  // key positions (0 for lanes without a pair) and the tagged-index base
  const bool act = (QC == 4) || (j < 4);
  const int koff = 4 * lg + jsel;
  const int lim = (act && qvalid) ? min(n_q, ke) : 0;
  const uint32_t lo_base = tagged_lo_base(qi);
  const size_t row_base = (size_t)b * p.T;
  auto qbuf = [&](int i) -> uint64_t* {
    return p.cand + ((row_base + t0 + i) * p.n_splits + split) * (size_t)p.cap;
  };

  int gcnt[QC];  // entries in each query's global buffer
#pragma unroll
  for (int i = 0; i < QC; ++i) gcnt[i] = 0;
  int stotal = 0;             // entries in the wave stage
  uint64_t th_lane = 0ull;    // own query's threshold: keep keys >= it
  const int limit = p.ksel + (p.cap - WSTG - p.ksel) / 2;

  // stage -> per-query buffers, each query's entries in stage (= key) order
  auto flush = [&]() {
    for (int e0 = 0; e0 < stotal; e0 += 64) {
      const int e = e0 + lane;
      const bool valid = e < stotal;
      const uint64_t v = valid ? stage[e] : 0ull;
      const int q = (int)(((uint32_t)v >> kTagShift) & 3u);
#pragma unroll
      for (int i = 0; i < QC; ++i) {
        const bool mine = valid && q == i;
        const uint64_t m = ballot64(mine);
        if (mine)
          qbuf(i)[gcnt[i] + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0))] = v;
        gcnt[i] += popc64(m);
      }
    }
    stotal = 0;
  };
  auto select_on = [&](uint64_t* buf, int n, int lim_kept) -> SelectResult {
    uint32_t mn, mx;
    wave_hi_range(buf, n, mn, mx);
    uint64_t prefix;
    int rem;
    select_start(mn, mx, prefix, rem);
    return wave_radix_select(buf, n, p.ksel, lim_kept, prefix, rem, hist);
  };

  // key rows of this sequence behind a bounds-checked buffer: rows >= kv_len read as 0
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(p.k + (size_t)b * p.S_max * DI, (uint32_t)kvl * DI);
  const int voff = r16 * DI + 32 * (DI == 128 ? lg : (lg & 1));

  i32x8 ring[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) ring[i] = load_key_tile(krs, voff + (ks + 16 * i) * DI);

  for (int s0 = ks; s0 < ke; s0 += 16 * PF) {
    float sc[PF];
#pragma unroll
    for (int ui = 0; ui < PF; ++ui) {
      sc[ui] = qo.template tile_score<EXACT>(ring[ui], p.g, jsel);
      ring[ui] = load_key_tile(krs, voff + (s0 + 16 * (ui + PF)) * DI);
    }
#pragma unroll
    for (int ui = 0; ui < PF; ++ui) {
      const int s = s0 + 16 * ui + koff;
      const uint64_t key = ((uint64_t)f32_to_ordered(sc[ui]) << 32) | (uint64_t)(lo_base - (uint32_t)s);
      const bool pass = (s < lim) & (key >= th_lane);
      const uint64_t bal = ballot64(pass);
      if (bal) {
        if (pass)
          stage[__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bal, stotal))] = key;
        stotal += popc64(bal);
      }
    }
    // the stage must take another block; each buffer must take a full stage
    if (stotal > WSTG - 64 * PF) {
      flush();
#pragma unroll
      for (int i = 0; i < QC; ++i) {
        if (gcnt[i] > p.cap - WSTG) {
          mem_fence_wave();
          uint64_t* buf = qbuf(i);
          const SelectResult sr = select_on(buf, gcnt[i], limit);
          gcnt[i] = wave_filter(buf, gcnt[i], sr.theta, [&](int pos, uint64_t v) { buf[pos] = v; });
          mem_fence_wave();
          if (qi == i) th_lane = sr.theta;
        }
      }
    }
  }

  // final exact selection for each query of the wave
  flush();
  mem_fence_wave();
#pragma unroll
  for (int i = 0; i < QC; ++i) {
    const int ti = t0 + i;
    if (ti >= p.T) break;
    uint64_t* buf = qbuf(i);
    const int n = gcnt[i];
    const uint64_t theta = (n > p.ksel) ? select_on(buf, n, 0).theta : 0ull;
    if (p.n_splits == 1) {
      // kept entries (ascending index) straight into the output row, then padding
      int32_t* orow = p.idx + (row_base + ti) * (size_t)p.ksel;
      float* srow = p.sel ? p.sel + (row_base + ti) * (size_t)p.ksel : nullptr;
      const int out = wave_filter(buf, n, theta, [&](int pos, uint64_t v) {
        orow[pos] = untag_index(v);
        if (srow) srow[pos] = ordered_to_f32((uint32_t)(v >> 32));
      });
      for (int pos = out + lane; pos < p.ksel; pos += 64) {
        orow[pos] = -1;
        if (srow) srow[pos] = -__builtin_inff();
      }
    } else {
      const int kept =
          (n > p.ksel) ? wave_filter(buf, n, theta, [&](int pos, uint64_t v) { buf[pos] = v; }) : n;
      if (lane == 0) p.cand_cnt[(row_base + ti) * p.n_splits + split] = kept;
    }
  }
}

// ------------------------------------------------------------------ merge of key splits

constexpr int kMergeBlock = 256;

__device__ __forceinline__ uint32_t block_reduce_minmax(uint32_t v, bool is_min, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = is_min ? wave_min_u32(v) : wave_max_u32(v);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  uint32_t r = red[0];
  for (int i = 1; i < kMergeBlock / 64; ++i) r = is_min ? min(r, red[i]) : max(r, red[i]);
  __syncthreads();
  return r;
}

// One block per query: union of the per-split lists (each ascending, splits in key
// order), exact top-k of the union, written in ascending index order.
__global__ __launch_bounds__(kMergeBlock) void ix_topk_merge_kernel(IxArgs p) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ int cnts[64];
  __shared__ uint32_t red[kMergeBlock / 64];
  __shared__ int pick[3];
  __shared__ int wave_cnt[kMergeBlock / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const size_t row = blockIdx.x;  // b * T + t
  const int NS = p.n_splits;
  for (int i = tid; i < NS; i += kMergeBlock) cnts[i] = p.cand_cnt[row * NS + i];
  __syncthreads();
  int N = 0;
  for (int i = 0; i < NS; ++i) N += cnts[i];
  const uint64_t* base = p.cand + row * NS * (size_t)p.cap;

  uint64_t theta = 0ull;
  if (N > p.ksel) {
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int i = 0; i < NS; ++i) {
      const uint64_t* sb = base + (size_t)i * p.cap;
      for (int e = tid; e < cnts[i]; e += kMergeBlock) {
        const uint32_t hi = (uint32_t)(sb[e] >> 32);
        mn = min(mn, hi);
        mx = max(mx, hi);
      }
    }
    mn = block_reduce_minmax(mn, true, red);
    mx = block_reduce_minmax(mx, false, red);
    uint64_t prefix;
    int rem;
    select_start(mn, mx, prefix, rem);
    uint32_t needed = (uint32_t)p.ksel;
    while (true) {
      const int dbits = rem < 8 ? rem : 8;
      const int shift = rem - dbits;
      const int nbins = 1 << dbits;
      const int hs = shift + dbits;
      for (int i = tid; i < kHistBins; i += kMergeBlock) hist[i] = 0u;
      __syncthreads();
      for (int i = 0; i < NS; ++i) {
        const uint64_t* sb = base + (size_t)i * p.cap;
        for (int e = tid; e < cnts[i]; e += kMergeBlock) {
          const uint64_t v = sb[e];
          if (hs >= 64 || (v >> hs) == prefix)
            atomicAdd(&hist[(uint32_t)(v >> shift) & (uint32_t)(nbins - 1)], 1u);
        }
      }
      __syncthreads();
      if (wid == 0) {
        int d;
        uint32_t above, c;
        wave_pick_digit(hist, nbins, needed, d, above, c);
        if (lane == 0) {
          pick[0] = d;
          pick[1] = (int)above;
          pick[2] = (int)c;
        }
      }
      __syncthreads();
      const int d = pick[0];
      const uint32_t above = (uint32_t)pick[1], c = (uint32_t)pick[2];
      __syncthreads();
      needed -= above;
      prefix = (prefix << dbits) | (uint64_t)d;
      rem = shift;
      if (c == needed || rem == 0) break;
    }
    theta = rem >= 64 ? 0ull : (prefix << rem);
  }

  // ordered write of the kept entries
  int32_t* orow = p.idx + row * (size_t)p.ksel;
  float* srow = p.sel ? p.sel + row * (size_t)p.ksel : nullptr;
  const uint64_t lt = lanemask_lt();
  int out = 0;
  for (int i = 0; i < NS; ++i) {
    const uint64_t* sb = base + (size_t)i * p.cap;
    const int ci = cnts[i];
    for (int e0 = 0; e0 < ci; e0 += kMergeBlock) {
      const int e = e0 + tid;
      const uint64_t v = e < ci ? sb[e] : 0ull;
      const bool keep = e < ci && v >= theta;
      const uint64_t bal = ballot64(keep);
      if (lane == 0) wave_cnt[wid] = popc64(bal);
      __syncthreads();
      int before = out;
      for (int w = 0; w < wid; ++w) before += wave_cnt[w];
      int total = 0;
      for (int w = 0; w < kMergeBlock / 64; ++w) total += wave_cnt[w];
      if (keep) {
        const int pos = before + popc64(bal & lt);
        orow[pos] = untag_index(v);
        if (srow) srow[pos] = ordered_to_f32((uint32_t)(v >> 32));
      }
      out += total;
      __syncthreads();
    }
  }
  for (int pos = out + tid; pos < p.ksel; pos += kMergeBlock) {
    orow[pos] = -1;
    if (srow) srow[pos] = -__builtin_inff();
  }
}

// ------------------------------------------------------------------ score rows (Stage 1 only)

template <int GMAX, int DI, bool EXACT>
__global__ __launch_bounds__(kBlock, 2) void ix_score_kernel(IxArgs p) {
  constexpr int QC = 4, HC = 4;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t u = (int64_t)blockIdx.x * kBlockWaves + wid;
  if (u >= p.units) return;
  const int b = (int)(u % p.B);
  const int qg = (int)(u / p.B);
  const int i0 = qg * QC;  // row within the window
  const int r16 = lane & 15, lg = lane >> 4;
  const int qi = r16 / HC, j = r16 % HC;
  const int jsel = j & 3;
  const int ri = i0 + qi;
  const bool qvalid = ri < p.rows;
  const int t = p.t_begin + ri;

  const int pos0 = p.q_pos0[b];
  int kvl = p.kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl > p.S_max ? p.S_max : kvl);
  const int n_q = qvalid ? visible_keys(pos0, kvl, t) : 0;

  QueryOperands<QC, GMAX, DI> qo;
  qo.load(p, b, t, qvalid, p.t_begin + i0, j, lg);

  const uint8_t* kbase = p.k + (size_t)b * p.S_max * DI;
  float* orow = p.scores + ((size_t)b * p.rows + (qvalid ? ri : 0)) * p.S_max;
  for (int s0 = 0; s0 < p.S_max; s0 += 16) {
    const int srow = min(s0 + r16, p.S_max - 1);
    const i32x8 a = load_row_slice<DI>(kbase + (size_t)srow * DI, lg);
    const float sc = qo.template tile_score<EXACT>(a, p.g, jsel);
    const int s = s0 + 4 * lg + jsel;
    if (qvalid && s < p.S_max) orow[s] = s < n_q ? sc + 0.0f : -__builtin_inff();
  }
}

template <typename F>
hipError_t dispatch_g(int g, F&& f) {
  if (g <= 1) return f(std::integral_constant<int, 1>{});
  if (g <= 2) return f(std::integral_constant<int, 2>{});
  if (g <= 4) return f(std::integral_constant<int, 4>{});
  if (g <= 8) return f(std::integral_constant<int, 8>{});
  return f(std::integral_constant<int, 16>{});
}

}  // namespace

// ------------------------------------------------------------------ host side

TopkPlan make_topk_plan(const ix_indexer_args& a, int k) {
  TopkPlan p{};
  p.qc = (a.T < 4 && a.H_I % 16 == 0) ? 1 : 4;
  p.hc = 16 / p.qc;
  p.g = a.H_I / p.hc;
  p.gmax = p.g <= 1 ? 1 : p.g <= 2 ? 2 : p.g <= 4 ? 4 : p.g <= 8 ? 8 : 16;
  p.qgroups = (a.T + p.qc - 1) / p.qc;
  const int64_t base_units = (int64_t)a.B * p.qgroups;
  int ns = 1;
  const int target = 2048;  // resident waves on 256 CUs at 2 waves per SIMD
  if (base_units < target) {
    const int64_t want = (target + base_units - 1) / base_units;
    int64_t by_len = a.S_max / 4096;
    if (by_len < 1) by_len = 1;
    ns = (int)(want < by_len ? want : by_len);
    if (ns > 64) ns = 64;
    if (ns < 1) ns = 1;
  }
  p.n_splits = ns;
  const int64_t sl = ((int64_t)a.S_max + ns - 1) / ns;
  p.split_len = (int)(((sl + 15) / 16) * 16);
  const int kpad = ((k + 63) / 64) * 64;
  p.cap = 2 * kpad + 1024;  // room for k, a full wave stage and slack
  p.units = base_units * ns;
  const size_t rows = (size_t)a.B * a.T * ns;
  p.cand_bytes = rows * (size_t)p.cap * sizeof(uint64_t);
  p.cnt_bytes = ((rows * sizeof(int32_t)) + 255) / 256 * 256;
  p.ws_bytes = p.cand_bytes + p.cnt_bytes;
  return p;
}

static IxArgs make_args(const ix_indexer_args& a) {
  IxArgs x{};
  x.q = a.q;
  x.k = a.k;
  x.w = a.w;
  x.q_pos0 = a.q_pos0;
  x.kv_len = a.kv_len;
  x.B = a.B;
  x.T = a.T;
  x.S_max = a.S_max;
  x.H_I = a.H_I;
  return x;
}

hipError_t launch_ix_topk(const ix_indexer_args& a, int k, const TopkPlan& pl, int32_t* idx,
                          float* sel_scores, void* ws, hipStream_t stream) {
  IxArgs x = make_args(a);
  x.g = pl.g;
  x.qgroups = pl.qgroups;
  x.n_splits = pl.n_splits;
  x.split_len = pl.split_len;
  x.cap = pl.cap;
  x.ksel = k;
  x.units = pl.units;
  x.cand = reinterpret_cast<uint64_t*>(ws);
  x.cand_cnt = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + pl.cand_bytes);
  x.idx = idx;
  x.sel = sel_scores;
  const dim3 grid((unsigned)((pl.units + kBlockWaves - 1) / kBlockWaves));
  const bool exact = pl.g == pl.gmax;
  hipError_t err = dispatch_g(pl.gmax, [&](auto GM) -> hipError_t {
    constexpr int G = decltype(GM)::value;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kBlock), 0, stream, x); };
    if (pl.qc == 4) {
      if (a.d_I == 128)
        exact ? go(ix_topk_partial_kernel<4, G, 128, true>) : go(ix_topk_partial_kernel<4, G, 128, false>);
      else
        exact ? go(ix_topk_partial_kernel<4, G, 64, true>) : go(ix_topk_partial_kernel<4, G, 64, false>);
    } else {
      if constexpr (G <= 4) {
        if (a.d_I == 128)
          exact ? go(ix_topk_partial_kernel<1, G, 128, true>) : go(ix_topk_partial_kernel<1, G, 128, false>);
        else
          exact ? go(ix_topk_partial_kernel<1, G, 64, true>) : go(ix_topk_partial_kernel<1, G, 64, false>);
      } else {
        return hipErrorInvalidValue;
      }
    }
    return hipGetLastError();
  });
  if (err != hipSuccess) return err;
  if (pl.n_splits > 1) {
    hipLaunchKernelGGL(ix_topk_merge_kernel, dim3((unsigned)((size_t)a.B * a.T)),
                       dim3(kMergeBlock), 0, stream, x);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_ix_score(const ix_indexer_args& a, int t_begin, int t_end, float* scores,
                           hipStream_t stream) {
  IxArgs x = make_args(a);
  const int rows = t_end - t_begin;
  x.g = a.H_I / 4;
  x.qgroups = (rows + 3) / 4;
  x.t_begin = t_begin;
  x.rows = rows;
  x.units = (int64_t)a.B * x.qgroups;
  x.scores = scores;
  const int gmax = x.g <= 1 ? 1 : x.g <= 2 ? 2 : x.g <= 4 ? 4 : x.g <= 8 ? 8 : 16;
  const dim3 grid((unsigned)((x.units + kBlockWaves - 1) / kBlockWaves));
  const bool exact = x.g == gmax;
  return dispatch_g(gmax, [&](auto GM) -> hipError_t {
    constexpr int G = decltype(GM)::value;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kBlock), 0, stream, x); };
    if (a.d_I == 128)
      exact ? go(ix_score_kernel<G, 128, true>) : go(ix_score_kernel<G, 128, false>);
    else
      exact ? go(ix_score_kernel<G, 64, true>) : go(ix_score_kernel<G, 64, false>);
    return hipGetLastError();
  });
}

}  // namespace ix
