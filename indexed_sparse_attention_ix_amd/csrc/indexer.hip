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
// (order preserved).  The threshold starts at an estimate from a sample (one hashed
// tile per stride group, scored first); a count check after the sweep proves it, or the
// sweep runs again from zero.  At the end an exact select leaves exactly
// min(k, count) entries, already in ascending index order, so no sort is needed.
//
// Key splits (small batches): each (query, split) keeps only its top-k' (k' <= k) and
// notes the smallest key it kept whenever it dropped any.  The merge takes the exact
// top-k of the union; that is the true top-k whenever every split that dropped keys
// kept nothing below the union's k-th key (all dropped keys then rank below it).
// Queries that fail the check are recomputed, still split, with every split keeping its
// exact top-k (then the union always holds the top-k); k' only trades merge work
// against how often that happens, never the result.
#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

constexpr int kBlockWaves = 4;
constexpr int kBlock = kBlockWaves * kWave;
constexpr int kHistBins = 256;
constexpr int kHistBatch = 4;    // 16-byte loads in flight per lane in a pass over a buffer
constexpr int kFinalBatch = 16;  // the same after the sweep, when the query operands are dead

// Key tiles in flight per wave: as many as the registers left beside the query operands
// allow (GMAX head blocks of 8 VGPRs each).  The wave's LDS stage takes two blocks of
// appends from every lane per tile in flight.
constexpr int prefetch_tiles(int gmax) { return gmax >= 16 ? 2 : gmax >= 8 ? 4 : 8; }
constexpr int wave_stage_entries(int gmax) { return 2 * 64 * prefetch_tiles(gmax); }

struct IxArgs {
  const uint8_t* q;
  const uint8_t* k;
  const float* w;
  const int32_t* q_pos0;
  const int32_t* kv_len;
  int B, T, S_max, H_I;
  int g;          // head blocks actually used (<= GMAX)
  int qgroups;    // query groups per sequence (over the row window for ix_score)
  int n_splits, split_len, cap;
  int ksel;       // entries each wave unit keeps (per split when n_splits > 1)
  int kout;       // k of the final selection (row width of idx)
  int fallback;   // 1: redo only the queries flagged in fb_flags (every split keeps k)
  int samp_tiles; // tiles in the threshold sample (0: no sampling)
  int pool;       // positions per key row (1: token keys; IndexPool: pooled block keys)
  int64_t units;
  int t_begin, rows;  // ix_score row window
  uint64_t* cand;
  int32_t* cand_cnt;
  uint64_t* split_min;  // per (query, split): smallest kept key if any key was dropped, else 0
  int32_t* fb_flags;    // per query: the merge could not prove its union held the top-k
  int32_t* idx;
  float* sel;
  float* scores;
  unsigned long long* dbg;  // debug status words (DebugWord), or null: no counting
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

// Keys (or pooled key blocks) visible to query t: unit j covers positions
// [pool*j, pool*j + pool) and is visible once its first position is (pool*j <= pos0 + t);
// kvl_units caps the count.  pool = 1 is the plain causal prefix.
__device__ __forceinline__ int visible_units(int pos0, int kvl_units, int t, int pool) {
  const long p = (long)pos0 + t;
  if (p < 0) return 0;
  const long v = p / pool + 1;
  return (int)(v > kvl_units ? kvl_units : v);
}

__device__ __forceinline__ int visible_keys(int pos0, int kvl, int t) {
  const long v = (long)pos0 + t + 1;
  return (int)(v < 0 ? 0 : (v > kvl ? kvl : v));
}

// Per-wave query operands: B operands for every head block and the matching weights.
//
// LIN (4 queries per wave, all 16 head blocks): the head sum is taken as
//   sum_h w_h max(0, x_h) = 1/2 sum_h w_h |x_h| + 1/2 sum_h w_h x_h,
// where the linear half is one more MFMA per key tile: sum_h w_h x_h = k . u with
// u = sum_h w_h q_h.  u is split into four e4m3 vectors with power-of-two scales,
// u ~= sum_j 2^E_j e_j (each term captures the next 4 significant bits of the residual;
// what the four leave is below 2^-16 of max|u|), and column (query, j) of the extra
// B operand holds e_j, so the head-sum reduction adds the four terms as it adds heads.
// That leaves one VALU op per head dot product (an FMA with an |x| source modifier)
// instead of two.  A key whose true score is 0 (every head dot product <= 0) would
// come out as rounding noise, so a visible key whose score is not above 1/16 of its
// |x| sum A is scored again the plain way in the same tile, which keeps exact zeros
// exact -- unless its query's threshold is already above A/8: its score, either way, is
// at most A/16 plus rounding error, far below A/8, so it cannot be kept.  That test needs
// w >= 0 (then A bounds the rounding of both halves): the kernels take this form only for
// waves whose queries' head weights are all >= 0, and the plain one otherwise.
template <int QC, int GMAX, int DI, bool LIN>
struct QueryOperands {
  i32x8 bq[GMAX];
  float wv[GMAX];  // LIN: w / 2
  i32x8 bl;        // LIN: e_j of the lane's (query, term j) column
  float sl;        // LIN: 2^E_j

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
        wv[g] = valid ? (LIN ? 0.5f : 1.f) * p.w[row] : 0.f;
      }
    }
    if constexpr (LIN) split_linear(j);
  }

  // u/2 over the lane's 32 depth elements (its lane group's slice) for query (lane&15)/4,
  // then the four terms; lane (query, j) keeps term j.
  __device__ __forceinline__ void split_linear(int j) {
    static_assert(QC == 4, "the linear terms fill the four columns of a query");
    float r[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) r[c] = 0.f;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
#pragma unroll
      for (int dw = 0; dw < 8; ++dw) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(bq[g][dw], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(bq[g][dw], true);
        r[4 * dw + 0] = fmaf(wv[g], lo[0], r[4 * dw + 0]);
        r[4 * dw + 1] = fmaf(wv[g], lo[1], r[4 * dw + 1]);
        r[4 * dw + 2] = fmaf(wv[g], hi[0], r[4 * dw + 2]);
        r[4 * dw + 3] = fmaf(wv[g], hi[1], r[4 * dw + 3]);
      }
    }
    // the quad's four lanes hold heads 4g + 0..3 of one query: add them (same bits in all four)
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      r[c] += dpp_f32<kDppQuadXor1>(r[c]);
      r[c] += dpp_f32<kDppQuadXor2>(r[c]);
    }
    i32x8 keep = {0, 0, 0, 0, 0, 0, 0, 0};
    float keep_scale = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float m = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) m = fmaxf(m, fabsf(r[c]));
      // the query's four lane groups hold the four depth slices
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      // scale 2^E with max|r| / 2^E in (224, 448]: m = f 2^e, f in [1, 2), 448 = 1.75 2^8.
      // Residuals below 2^-100 are dropped.
      const uint32_t mb = __builtin_bit_cast(uint32_t, m);
      const bool live = m >= 0x1p-100f;
      const int e = (int)(mb >> 23) - 127;
      const int E = e - ((mb & 0x7FFFFFu) <= 0x600000u ? 8 : 7);
      const float scale = live ? __builtin_bit_cast(float, (uint32_t)(E + 127) << 23) : 0.f;
      const float inv = live ? __builtin_bit_cast(float, (uint32_t)(127 - E) << 23) : 0.f;
#pragma unroll
      for (int dw = 0; dw < 8; ++dw) {
        // |r * inv| <= 448: round to nearest e4m3, then take the rounded value off the
        // residual (exact: the difference is representable in fp32)
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * dw + 0] * inv, r[4 * dw + 1] * inv, 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * dw + 2] * inv, r[4 * dw + 3] * inv, pk, true);
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(pk, true);
        r[4 * dw + 0] = fmaf(-scale, lo[0], r[4 * dw + 0]);
        r[4 * dw + 1] = fmaf(-scale, lo[1], r[4 * dw + 1]);
        r[4 * dw + 2] = fmaf(-scale, hi[0], r[4 * dw + 2]);
        r[4 * dw + 3] = fmaf(-scale, hi[1], r[4 * dw + 3]);
        if (jj == j) keep[dw] = pk;
      }
      if (jj == j) keep_scale = scale;
    }
    bl = keep;
    sl = keep_scale;
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
  static __device__ __forceinline__ void accumulate_abs(f32x4& acc, const f32x4& x, float w) {
    acc[0] = fmaf(w, fabsf(x[0]), acc[0]);
    acc[1] = fmaf(w, fabsf(x[1]), acc[1]);
    acc[2] = fmaf(w, fabsf(x[2]), acc[2]);
    acc[3] = fmaf(w, fabsf(x[3]), acc[3]);
  }

  // Sum of the HC adjacent columns of one query: lane l ends up with key
  // 4*(l>>4) + (j & 3) and query (l & 15) / HC, where j = (l & 15) % HC; for HC = 16
  // only lanes with j < 4 carry a distinct pair.
  static __device__ __forceinline__ float head_sum(const f32x4& acc, int jsel) {
    constexpr int HC = 16 / QC;
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

  // Score of one (query, key) pair per lane for the 16-key tile held in `a` (pair as in
  // head_sum).  EXACT: all GMAX head blocks are used; the MFMA of block g+1 is issued
  // before the epilogue of block g so that the matrix core and the VALU overlap.
  // `need`: the lane's key is visible to its query; `th_hi`: the high word of the query's
  // threshold key (0: none yet).  LIN rescoring looks only at keys that could be kept.
  template <bool EXACT>
  __device__ __forceinline__ float tile_score(const i32x8& a, int g_rt, int jsel, bool need,
                                              uint32_t th_hi) const {
    if constexpr (LIN) {
      static_assert(EXACT, "the linear form uses every head block");
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      f32x4 x = mfma_e4m3_16x16x128(a, bq[0]);
#pragma unroll
      for (int g = 1; g < GMAX; ++g) {
        const f32x4 y = mfma_e4m3_16x16x128(a, bq[g]);
        accumulate_abs(acc, x, wv[g - 1]);
        x = y;
      }
      const f32x4 l = mfma_e4m3_16x16x128(a, bl);
      accumulate_abs(acc, x, wv[GMAX - 1]);
      const f32x4 lin = {l[0] * sl, l[1] * sl, l[2] * sl, l[3] * sl};
      const float ah = head_sum(acc, jsel);  // 1/2 sum_h w_h |x_h|
      float s = ah + head_sum(lin, jsel);    // + 1/2 sum_h w_h x_h
      const bool again = need && !(s > 0.125f * ah) && th_hi <= f32_to_ordered(0.25f * ah);
      if (ballot64(again)) {
        const float e = 2.f * plain_score(a, jsel);
        s = again ? e : s;
      }
      return s;
    } else if constexpr (EXACT) {
      return plain_score(a, jsel);
    } else {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g < g_rt) accumulate(acc, mfma_e4m3_16x16x128(a, bq[g]), wv[g]);
      }
      return head_sum(acc, jsel);
    }
  }

  // sum_h wv_h max(0, x_h) over all GMAX head blocks
  __device__ __forceinline__ float plain_score(const i32x8& a, int jsel) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f32x4 x = mfma_e4m3_16x16x128(a, bq[0]);
#pragma unroll
    for (int g = 1; g < GMAX; ++g) {
      const f32x4 y = mfma_e4m3_16x16x128(a, bq[g]);
      accumulate(acc, x, wv[g - 1]);
      x = y;
    }
    accumulate(acc, x, wv[GMAX - 1]);
    return head_sum(acc, jsel);
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
// NB chunks are loaded before any is counted, so the L2 latency is paid once per
// 128 * NB entries.
template <int NB>
__device__ void wave_hist(const uint64_t* buf, int n, uint64_t prefix, int hs, int shift,
                          uint32_t dmask, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  for (int e0 = 0; e0 < n; e0 += 128 * NB) {
    uint64_t x[NB][2];
#pragma unroll
    for (int u = 0; u < NB; ++u) load_pair(buf, e0 + 128 * u + 2 * lane, n, x[u][0], x[u][1]);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
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
template <int NB>
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
    wave_hist<NB>(buf, n, prefix, rem, shift, (uint32_t)(nbins - 1), hist);
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
template <int NB, typename Out>
__device__ int wave_filter(const uint64_t* buf, int n, uint64_t theta, Out&& out) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lanemask_lt();
  int total = 0;
  for (int e0 = 0; e0 < n; e0 += 128 * NB) {
    uint64_t x[NB][2];
#pragma unroll
    for (int u = 0; u < NB; ++u) load_pair(buf, e0 + 128 * u + 2 * lane, n, x[u][0], x[u][1]);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
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

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o < v ? o : v;
  }
  return v;
}

// Smallest entry of buf[0, n) (n > 0), wave-reduced.
__device__ uint64_t wave_min_key(const uint64_t* buf, int n) {
  const int lane = threadIdx.x & 63;
  uint64_t m = ~0ull;
  for (int e = 2 * lane; e < n; e += 128) {
    uint64_t x0, x1;
    load_pair(buf, e, n, x0, x1);
    m = x0 < m ? x0 : m;
    if (e + 1 < n) m = x1 < m ? x1 : m;
  }
  return wave_min_u64(m);
}

// s_waitcnt immediate that waits for this wave's vector-memory operations only (vmcnt 0,
// expcnt and lgkmcnt at their maxima: no wait on those)
constexpr int kWaitVmemOnly = 0x0F70;

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
template <int NB>
__device__ void wave_hi_range(const uint64_t* buf, int n, uint32_t& mn, uint32_t& mx) {
  const int lane = threadIdx.x & 63;
  mn = 0xFFFFFFFFu;
  mx = 0u;
  for (int e0 = 0; e0 < n; e0 += 128 * NB) {
    uint64_t x[NB][2];
#pragma unroll
    for (int u = 0; u < NB; ++u) load_pair(buf, e0 + 128 * u + 2 * lane, n, x[u][0], x[u][1]);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
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

// Whether every head weight of query rows [t0, min(t0 + 4, t_end)) of sequence b is >= 0;
// the same answer in every lane.  A wave's four queries share one scoring form, so with
// mixed-sign weights a query's scores depend on its neighbours' weights through that choice
// (both forms stay within the same error bound).
__device__ __forceinline__ bool weights_nonneg(const IxArgs& p, int b, int t0, int t_end) {
  bool neg = false;
  for (int e = (int)(threadIdx.x & 63); e < 4 * p.H_I; e += 64) {
    const int t = t0 + e / p.H_I;
    if (t < t_end) neg |= p.w[((size_t)b * p.T + t) * p.H_I + e % p.H_I] < 0.f;
  }
  return ballot64(neg) == 0;
}

template <int QC, int GMAX, int DI, bool EXACT, bool LIN>
__device__ __forceinline__ void topk_partial_body(const IxArgs& p, int64_t u, int split, int b,
                                                  int t0, uint32_t* hist, uint64_t* stage) {
  constexpr int HC = 16 / QC;
  // key tiles in flight per wave (the 16-block case keeps 128 VGPRs of query operands)
  constexpr int PF = prefetch_tiles(GMAX);
  constexpr int WSTG = wave_stage_entries(GMAX);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, lg = lane >> 4;
  const int qi = r16 / HC, j = r16 % HC;
  const int jsel = j & 3;
  const int t = t0 + qi;
  const bool qvalid = t < p.T;
  if (p.fallback) {
    bool redo = false;
#pragma unroll
    for (int i = 0; i < QC; ++i)
      if (t0 + i < p.T && p.fb_flags[(size_t)b * p.T + t0 + i]) redo = true;
    if (!redo) return;
  }

  const int pos0 = p.q_pos0[b];
  // key rows here are units of `pool` positions (1: tokens); kv_len counts positions
  const int pool = p.pool;
  int kvl = p.kv_len[b];
  kvl = kvl < 0 ? 0 : (kvl + pool - 1) / pool;
  kvl = kvl > p.S_max ? p.S_max : kvl;
  const int n_q = qvalid ? visible_units(pos0, kvl, t, pool) : 0;
  const int t_last = (t0 + QC < p.T ? t0 + QC : p.T) - 1;
  const int n_max = visible_units(pos0, kvl, t_last, pool);
  const int ks = split * p.split_len;
  const int ke = min(ks + p.split_len, n_max);

  QueryOperands<QC, GMAX, DI, LIN> qo;
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

  int gcnt[QC];         // entries in each query's global buffer
  uint32_t dropped = 0;  // bit i: a compaction removed entries from query i's buffer
#pragma unroll
  for (int i = 0; i < QC; ++i) gcnt[i] = 0;
  int stotal = 0;             // entries in the wave stage
  uint64_t th_lane = 0ull;    // own query's threshold: keep keys >= it
  const int limit = p.ksel + (p.cap - WSTG - p.ksel) / 2;

  // stage -> per-query buffers, each query's entries in stage (= key) order.  The buffers
  // are sized so that a flush always fits (a compaction follows any flush that leaves less
  // than a stage of room); entries that would not fit are dropped, not written, and counted
  // in the debug status.
  auto flush = [&]() {
    int lost = 0;
    for (int e0 = 0; e0 < stotal; e0 += 64) {
      const int e = e0 + lane;
      const bool valid = e < stotal;
      const uint64_t v = valid ? stage[e] : 0ull;
      const int q = (int)(((uint32_t)v >> kTagShift) & 3u);
#pragma unroll
      for (int i = 0; i < QC; ++i) {
        const bool mine = valid && q == i;
        const uint64_t m = ballot64(mine);
        const int pos = gcnt[i] + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (mine && pos < p.cap) qbuf(i)[pos] = v;
        const int n = gcnt[i] + popc64(m);
        lost += n > p.cap ? n - max(gcnt[i], p.cap) : 0;
        gcnt[i] = min(n, p.cap);
      }
    }
    stotal = 0;
    if (lost && p.dbg && lane == 0) atomicAdd(p.dbg + kDbgTopkOverflow, (unsigned long long)lost);
  };
  auto select_on = [&](auto nb, uint64_t* buf, int n, int kk, int lim_kept) -> SelectResult {
    constexpr int NB = decltype(nb)::value;
    uint32_t mn, mx;
    wave_hi_range<NB>(buf, n, mn, mx);
    uint64_t prefix;
    int rem;
    select_start(mn, mx, prefix, rem);
    return wave_radix_select<NB>(buf, n, kk, lim_kept, prefix, rem, hist);
  };
  using SweepBatch = std::integral_constant<int, kHistBatch>;
  using FinalBatch = std::integral_constant<int, kFinalBatch>;
  // visible keys of query slot i inside this unit's key range
  auto unit_keys = [&](int i) -> int {
    if (t0 + i >= p.T) return 0;
    const int n = min(visible_units(pos0, kvl, t0 + i, pool), ke) - ks;
    return n > 0 ? n : 0;
  };

  // key rows of this sequence behind a bounds-checked buffer: rows >= kv_len read as 0
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(p.k + (size_t)b * p.S_max * DI, (uint32_t)kvl * DI);
  const int voff = r16 * DI + 32 * (DI == 128 ? lg : (lg & 1));

  // Scores tiles base + 16 * step * jj (jj < count) of the unit, PF tiles in flight, and
  // appends every visible key >= the lane's threshold; buffers that near capacity are
  // compacted to a threshold that keeps at least k' entries.
  auto sweep = [&](int base, int step, int count) __attribute__((always_inline)) {
    // tile jj of the sweep: jj itself (step 1), or a hashed tile inside stride group jj, so
    // that a sample cannot alias with periodic structure in the keys
    auto tile_idx = [&](int jj) {
      return step * jj + (step > 1 ? (int)((((uint32_t)jj * 2654435761u) >> 16) % (uint32_t)step) : 0);
    };
    auto tile_off = [&](int jj) { return voff + min(base + 16 * tile_idx(jj), kvl) * DI; };
    // One-query units (decode) run one wave per SIMD, so no other wave covers this one's
    // memory waits: the tiles are scored and refilled strictly in ring order (scheduling
    // barriers), so the wait for a tile leaves the other PF - 1 in flight.  Left free, the
    // scheduler interleaves all PF tiles' products at the top of the ring and sinks their
    // refills to the bottom, and every step waits for the whole ring.
    i32x8 ring[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      ring[i] = load_key_tile(krs, tile_off(i));
      if constexpr (QC == 1) __builtin_amdgcn_sched_barrier(0);
    }
    for (int j0 = 0; j0 < count; j0 += PF) {
      float sc[PF];
#pragma unroll
      for (int ui = 0; ui < PF; ++ui) {
        const bool need = (j0 + ui < count) & (base + 16 * tile_idx(j0 + ui) + koff < lim);
        sc[ui] = qo.template tile_score<EXACT>(ring[ui], p.g, jsel, need, (uint32_t)(th_lane >> 32));
        ring[ui] = load_key_tile(krs, tile_off(j0 + ui + PF));
        if constexpr (QC == 1) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int ui = 0; ui < PF; ++ui) {
        const int s = base + 16 * tile_idx(j0 + ui) + koff;
        const uint64_t key =
            ((uint64_t)f32_to_ordered(sc[ui]) << 32) | (uint64_t)(lo_base - (uint32_t)s);
        const bool pass = (j0 + ui < count) & (s < lim) & (key >= th_lane);
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
            const SelectResult sr = select_on(SweepBatch{}, buf, gcnt[i], p.ksel, limit);
            gcnt[i] = wave_filter<kHistBatch>(buf, gcnt[i], sr.theta,
                                              [&](int pos, uint64_t v) { buf[pos] = v; });
            mem_fence_wave();
            dropped |= 1u << i;
            if (qi == i) th_lane = sr.theta;
            if (p.dbg && lane == 0) atomicAdd(p.dbg + kDbgTopkCompactions, 1ull);
          }
        }
        // Vector loads and stores complete in order under one counter, and the flush stores
        // a count of entries no one knows in advance: without a wait here the wait for the
        // next step's first tile could not be counted and would take every tile in flight.
        // This branch is rare; waiting in it keeps the other tiles' loads in flight.
        __builtin_amdgcn_s_waitcnt(kWaitVmemOnly);
      }
    }
    flush();
    mem_fence_wave();
  };

  // Sampled starting threshold: score a 1/stride share of the unit's tiles first (stride >= 4,
  // at most samp_tiles tiles) and start each query at the r-th best sampled key, r a few
  // standard deviations above the number of the query's top-k' keys the sample is expected
  // to hold.  That is a guess; the check after the sweep keeps the result exact.
  //  * 4-query units: one hashed tile of every stride group, scored again by the sweep (the
  //    query groups of a sequence share their key rows, so the second read hits the caches);
  //  * 1-query units (decode): each unit reads its keys alone, so a second read would come
  //    from memory.  The sample is the unit's first tiles instead: their entries stay in
  //    the buffer, filtered by the threshold (order kept), and the sweep goes on after them.
  const int n_tiles = ke > ks ? (ke - ks + 15) / 16 : 0;
  const int stride = p.samp_tiles > 0 ? n_tiles / p.samp_tiles : 0;
  int first = 0;  // tiles already swept
  if (stride >= 4) {
    if constexpr (QC == 1) {
      sweep(ks, 1, p.samp_tiles);
      first = p.samp_tiles;
    } else {
      sweep(ks, stride, p.samp_tiles);
    }
#pragma unroll
    for (int i = 0; i < QC; ++i) {
      const int keff = min(p.ksel, unit_keys(i));
      const float c = (float)keff / (float)stride;
      const int rank = (int)ceilf(c + 4.f * sqrtf(c)) + 1;
      uint64_t th = 0ull;
      if (rank < gcnt[i]) {
        th = select_on(SweepBatch{}, qbuf(i), gcnt[i], rank, 0).theta;
        dropped |= 1u << i;
        if constexpr (QC == 1) {
          uint64_t* buf = qbuf(i);
          gcnt[i] = wave_filter<kHistBatch>(buf, gcnt[i], th,
                                            [&](int pos, uint64_t v) { buf[pos] = v; });
        }
      }
      if (qi == i) th_lane = th;
      if constexpr (QC != 1) gcnt[i] = 0;
    }
    mem_fence_wave();
  }
  sweep(ks + 16 * first, 1, n_tiles - first);
  // Every query must end with at least min(k', visible) entries, which proves that its
  // k'-th key is at or above its starting threshold; otherwise sweep again from zero.
  bool short_q = false;
#pragma unroll
  for (int i = 0; i < QC; ++i) short_q |= gcnt[i] < min(p.ksel, unit_keys(i));
  if (short_q) {
    if (p.dbg && lane == 0) atomicAdd(p.dbg + kDbgTopkResweeps, 1ull);
#pragma unroll
    for (int i = 0; i < QC; ++i) gcnt[i] = 0;
    dropped = 0;
    th_lane = 0ull;
    sweep(ks, 1, n_tiles);
  }

  // final exact selection for each query of the wave
#pragma unroll
  for (int i = 0; i < QC; ++i) {
    const int ti = t0 + i;
    if (ti >= p.T) break;
    uint64_t* buf = qbuf(i);
    const int n = gcnt[i];
    const uint64_t theta = (n > p.ksel) ? select_on(FinalBatch{}, buf, n, p.ksel, 0).theta : 0ull;
    if (p.n_splits == 1) {
      // kept entries (ascending index) straight into the output row, then padding
      int32_t* orow = p.idx + (row_base + ti) * (size_t)p.kout;
      float* srow = p.sel ? p.sel + (row_base + ti) * (size_t)p.kout : nullptr;
      const int out = wave_filter<kFinalBatch>(buf, n, theta, [&](int pos, uint64_t v) {
        orow[pos] = untag_index(v);
        if (srow) srow[pos] = ordered_to_f32((uint32_t)(v >> 32));
      });
      for (int pos = out + lane; pos < p.kout; pos += 64) {
        orow[pos] = -1;
        if (srow) srow[pos] = -__builtin_inff();
      }
    } else {
      const int kept =
          (n > p.ksel) ? wave_filter<kFinalBatch>(buf, n, theta,
                                                  [&](int pos, uint64_t v) { buf[pos] = v; })
                       : n;
      uint64_t low = 0ull;
      if ((((dropped >> i) & 1u) || n > p.ksel) && kept > 0) {
        mem_fence_wave();
        low = wave_min_key(buf, kept);
      }
      if (lane == 0) {
        p.cand_cnt[(row_base + ti) * p.n_splits + split] = kept;
        p.split_min[(row_base + ti) * p.n_splits + split] = low;
      }
    }
  }
}

template <int QC, int GMAX, int DI, bool EXACT>
__global__ __launch_bounds__(kBlock, 2) void ix_topk_partial_kernel(IxArgs p) {
  constexpr int WSTG = wave_stage_entries(GMAX);
  __shared__ uint32_t hist_all[kBlockWaves][kHistBins];
  __shared__ uint64_t stage_all[kBlockWaves][WSTG];
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t u = (int64_t)blockIdx.x * kBlockWaves + wid;
  if (u >= p.units) return;
  const int split = (int)(u % p.n_splits);
  const int64_t r = u / p.n_splits;
  const int b = (int)(r % p.B);
  const int qg = p.qgroups - 1 - (int)(r / p.B);  // latest (heaviest) query groups first
  const int t0 = qg * QC;
  // the |x| + linear-MFMA form at 4 queries and 64 heads when the weights allow it
  if constexpr (QC == 4 && GMAX == 16 && EXACT) {
    if (weights_nonneg(p, b, t0, p.T)) {
      topk_partial_body<QC, GMAX, DI, EXACT, true>(p, u, split, b, t0, hist_all[wid], stage_all[wid]);
      return;
    }
  }
  topk_partial_body<QC, GMAX, DI, EXACT, false>(p, u, split, b, t0, hist_all[wid], stage_all[wid]);
}

// ------------------------------------------------------------------ merge of key splits

constexpr int kMergeBlock = 512;
constexpr int kMergeWaves = kMergeBlock / 64;

__device__ __forceinline__ uint32_t block_reduce_minmax(uint32_t v, bool is_min, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = is_min ? wave_min_u32(v) : wave_max_u32(v);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  uint32_t r = red[0];
  for (int i = 1; i < kMergeWaves; ++i) r = is_min ? min(r, red[i]) : max(r, red[i]);
  __syncthreads();
  return r;
}

// One block per query: union of the per-split lists (each ascending, splits in key
// order), exact top-k of the union, written in ascending index order.  Also decides
// whether the union provably held the true top-k (see the file header) and flags the
// query for the unsplit pass if not.  The lists are walked as one flat range of
// n_splits * ksel slots (slot j of split i valid when j < count_i).  When the slots fit
// (dynamic LDS of 8 bytes per slot), they are copied to LDS once and every pass reads
// them there (an empty slot holds 0, which no key equals); otherwise each pass reads
// them from memory with several loads in flight.
constexpr int kMergeLdsSlots = 12288;
__global__ __launch_bounds__(kMergeBlock) void ix_topk_merge_kernel(IxArgs p) {
  extern __shared__ uint64_t lds_slots[];
  __shared__ uint32_t hist[kHistBins];
  __shared__ int cnts[64];
  __shared__ uint64_t smin[64];
  __shared__ uint32_t red[kMergeWaves];
  __shared__ uint64_t red64[kMergeWaves];
  __shared__ int pick[3];
  __shared__ int wave_cnt[kMergeWaves];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const size_t row = blockIdx.x;  // b * T + t
  if (p.fallback && !p.fb_flags[row]) return;  // whole block: row is per block
  const int NS = p.n_splits;
  for (int i = tid; i < NS; i += kMergeBlock) {
    cnts[i] = p.cand_cnt[row * NS + i];
    smin[i] = p.split_min[row * NS + i];
  }
  __syncthreads();
  int N = 0;
  uint64_t trunc_max = 0ull;  // largest "smallest kept key" over splits that dropped keys
  for (int i = 0; i < NS; ++i) {
    N += cnts[i];
    trunc_max = smin[i] > trunc_max ? smin[i] : trunc_max;
  }
  const uint64_t* base = p.cand + row * NS * (size_t)p.cap;
  const int per = p.ksel;      // slots per split
  const int P = NS * per;      // padded slot count
  const bool in_lds = P <= kMergeLdsSlots;
  auto mem_slot = [&](int e, uint64_t& v) -> bool {
    if (e >= P) return false;
    const int i = e / per, j = e - i * per;
    if (j >= cnts[i]) return false;
    v = base[(size_t)i * p.cap + j];
    return true;
  };
  if (in_lds) {
    for (int e0 = 0; e0 < P; e0 += 4 * kMergeBlock) {
      uint64_t v[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) ok[u] = mem_slot(e0 + u * kMergeBlock + tid, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kMergeBlock + tid;
        if (e < P) lds_slots[e] = ok[u] ? v[u] : 0ull;
      }
    }
    __syncthreads();
  }
  auto slot = [&](int e, uint64_t& v) -> bool {
    if (!in_lds) return mem_slot(e, v);
    if (e >= P) return false;
    v = lds_slots[e];
    return v != 0ull;
  };

  uint64_t theta = 0ull;
  if (N > p.kout) {
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int e0 = 0; e0 < P; e0 += 4 * kMergeBlock) {
      uint64_t v[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) ok[u] = slot(e0 + u * kMergeBlock + tid, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (ok[u]) {
          mn = min(mn, (uint32_t)(v[u] >> 32));
          mx = max(mx, (uint32_t)(v[u] >> 32));
        }
      }
    }
    mn = block_reduce_minmax(mn, true, red);
    mx = block_reduce_minmax(mx, false, red);
    uint64_t prefix;
    int rem;
    select_start(mn, mx, prefix, rem);
    uint32_t needed = (uint32_t)p.kout;
    while (true) {
      const int dbits = rem < 8 ? rem : 8;
      const int shift = rem - dbits;
      const int nbins = 1 << dbits;
      const int hs = shift + dbits;
      for (int i = tid; i < kHistBins; i += kMergeBlock) hist[i] = 0u;
      __syncthreads();
      for (int e0 = 0; e0 < P; e0 += 4 * kMergeBlock) {
        uint64_t v[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ok[u] = slot(e0 + u * kMergeBlock + tid, v[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (ok[u] && (hs >= 64 || (v[u] >> hs) == prefix))
            atomicAdd(&hist[(uint32_t)(v[u] >> shift) & (uint32_t)(nbins - 1)], 1u);
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

  // ordered write of the kept entries (slot order is split order, then list order)
  int32_t* orow = p.idx + row * (size_t)p.kout;
  float* srow = p.sel ? p.sel + row * (size_t)p.kout : nullptr;
  const uint64_t lt = lanemask_lt();
  int out = 0;
  uint64_t kept_min = ~0ull;
  for (int e0 = 0; e0 < P; e0 += kMergeBlock) {
    uint64_t v = 0ull;
    const bool keep = slot(e0 + tid, v) && v >= theta;
    const uint64_t bal = ballot64(keep);
    if (lane == 0) wave_cnt[wid] = popc64(bal);
    __syncthreads();
    int before = out, total = 0;
    for (int w = 0; w < kMergeWaves; ++w) {
      before += w < wid ? wave_cnt[w] : 0;
      total += wave_cnt[w];
    }
    if (keep) {
      const int pos = before + popc64(bal & lt);
      orow[pos] = untag_index(v);
      if (srow) srow[pos] = ordered_to_f32((uint32_t)(v >> 32));
      kept_min = v < kept_min ? v : kept_min;
    }
    out += total;
    __syncthreads();
  }
  for (int pos = out + tid; pos < p.kout; pos += kMergeBlock) {
    orow[pos] = -1;
    if (srow) srow[pos] = -__builtin_inff();
  }
  if (p.fb_flags && !p.fallback) {
    // k-th key of the union = smallest kept entry (when the union has >= k entries)
    kept_min = wave_min_u64(kept_min);
    if (lane == 0) red64[wid] = kept_min;
    __syncthreads();
    if (tid == 0) {
      uint64_t kth = red64[0];
      for (int w = 1; w < kMergeWaves; ++w) kth = red64[w] < kth ? red64[w] : kth;
      const bool proven = trunc_max == 0ull || (N >= p.kout && trunc_max <= kth);
      p.fb_flags[row] = proven ? 0 : 1;
      if (!proven && p.dbg) atomicAdd(p.dbg + kDbgTopkSplitRecomputes, 1ull);
    }
  }
}

// ------------------------------------------------------------------ score rows (Stage 1 only)

template <int GMAX, int DI, bool EXACT, bool LIN>
__device__ __forceinline__ void score_body(const IxArgs& p, int b, int i0) {
  constexpr int QC = 4, HC = 4;
  const int lane = threadIdx.x & 63;
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

  QueryOperands<QC, GMAX, DI, LIN> qo;
  qo.load(p, b, t, qvalid, p.t_begin + i0, j, lg);

  const uint8_t* kbase = p.k + (size_t)b * p.S_max * DI;
  float* orow = p.scores + ((size_t)b * p.rows + (qvalid ? ri : 0)) * p.S_max;
  for (int s0 = 0; s0 < p.S_max; s0 += 16) {
    const int srow = min(s0 + r16, p.S_max - 1);
    const i32x8 a = load_row_slice<DI>(kbase + (size_t)srow * DI, lg);
    const int s = s0 + 4 * lg + jsel;
    const float sc = qo.template tile_score<EXACT>(a, p.g, jsel, qvalid && s < n_q, 0u);
    if (qvalid && s < p.S_max) orow[s] = s < n_q ? sc + 0.0f : -__builtin_inff();
  }
}

template <int GMAX, int DI, bool EXACT>
__global__ __launch_bounds__(kBlock, 2) void ix_score_kernel(IxArgs p) {
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t u = (int64_t)blockIdx.x * kBlockWaves + wid;
  if (u >= p.units) return;
  const int b = (int)(u % p.B);
  const int i0 = (int)(u / p.B) * 4;  // row within the window
  if constexpr (GMAX == 16 && EXACT) {
    if (weights_nonneg(p, b, p.t_begin + i0, p.t_begin + p.rows)) {
      score_body<GMAX, DI, EXACT, true>(p, b, i0);
      return;
    }
  }
  score_body<GMAX, DI, EXACT, false>(p, b, i0);
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
  // waves to aim for: two per SIMD for the MFMA-bound 4-query kernel; the 1-query (decode)
  // kernel streams keys and does better with half as many, twice as long splits (its
  // threshold sample then kicks in and the merge has fewer lists)
  const int target = p.qc == 1 ? 1024 : 2048;
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
  // With many splits each keeps about twice its even share of the top-k (at least 256);
  // the merge proves or refutes that this was enough.
  int ks = k;
  if (ns > 1) {
    const int share = ((2 * ((k + ns - 1) / ns) + 63) / 64) * 64;
    ks = share > 256 ? share : 256;
    if (ks > k) ks = k;
  }
  p.ksplit = ks;
  const int kspad = ((ks + 63) / 64) * 64;
  // room for k', a full wave stage and slack for a run of appends between compactions
  const int stage = wave_stage_entries(p.gmax);
  const int slack = 2 * stage > 1024 ? 2 * stage : 1024;
  p.cap = 2 * kspad + slack;
  p.fb_cap = 2 * kpad + slack;
  // a threshold sample must fit a candidate buffer without a compaction
  // (the 1-query decode kernel reads its sample from memory a second time: a smaller one)
  const int samp_max = p.qc == 1 ? 32 : 64;
  auto samp = [&](int cap) { const int t = (cap - stage) / 16; return t < samp_max ? t : samp_max; };
  p.samp_tiles = samp(p.cap);
  p.fb_samp_tiles = samp(p.fb_cap);
  p.units = base_units * ns;
  const size_t qrows = (size_t)a.B * a.T;
  const size_t rows = qrows * ns;
  size_t cand = rows * (size_t)p.cap;
  if (ks < k && rows * (size_t)p.fb_cap > cand) cand = rows * (size_t)p.fb_cap;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  p.cand_bytes = up(cand * sizeof(uint64_t));
  p.cnt_bytes = up(rows * sizeof(int32_t));
  p.min_bytes = up(rows * sizeof(uint64_t));
  p.flag_bytes = up(qrows * sizeof(int32_t));
  p.ws_bytes = p.cand_bytes + p.cnt_bytes + p.min_bytes + p.flag_bytes;
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
                          float* sel_scores, void* ws, hipStream_t stream, int pool,
                          unsigned long long* dbg) {
  IxArgs x = make_args(a);
  x.dbg = dbg;
  x.g = pl.g;
  x.qgroups = pl.qgroups;
  x.n_splits = pl.n_splits;
  x.split_len = pl.split_len;
  x.cap = pl.cap;
  x.ksel = pl.ksplit;
  x.kout = k;
  x.fallback = 0;
  x.samp_tiles = pl.samp_tiles;
  x.pool = pool;
  x.units = pl.units;
  char* w = reinterpret_cast<char*>(ws);
  x.cand = reinterpret_cast<uint64_t*>(w);
  x.cand_cnt = reinterpret_cast<int32_t*>(w + pl.cand_bytes);
  x.split_min = reinterpret_cast<uint64_t*>(w + pl.cand_bytes + pl.cnt_bytes);
  x.fb_flags = pl.ksplit < k
                   ? reinterpret_cast<int32_t*>(w + pl.cand_bytes + pl.cnt_bytes + pl.min_bytes)
                   : nullptr;
  x.idx = idx;
  x.sel = sel_scores;
  const bool exact = pl.g == pl.gmax;
  auto partial = [&](const IxArgs& xa) -> hipError_t {
    const dim3 grid((unsigned)((xa.units + kBlockWaves - 1) / kBlockWaves));
    return dispatch_g(pl.gmax, [&](auto GM) -> hipError_t {
    constexpr int G = decltype(GM)::value;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kBlock), 0, stream, xa); };
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
  };
  hipError_t err = partial(x);
  if (err != hipSuccess || pl.n_splits == 1) return err;
  auto merge = [&](const IxArgs& xa) -> hipError_t {
    const int slots = xa.n_splits * xa.ksel;
    const size_t lds = slots <= kMergeLdsSlots ? (size_t)slots * sizeof(uint64_t) : 0;
    if (lds > 48 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(ix_topk_merge_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(ix_topk_merge_kernel, dim3((unsigned)((size_t)a.B * a.T)),
                       dim3(kMergeBlock), lds, stream, xa);
    return hipGetLastError();
  };
  err = merge(x);
  if (err != hipSuccess || !x.fb_flags) return err;
  // the flagged queries again, every split keeping its exact top-k (the other waves and
  // merge blocks exit at once)
  IxArgs f = x;
  f.fallback = 1;
  f.cap = pl.fb_cap;
  f.ksel = k;
  f.samp_tiles = pl.fb_samp_tiles;
  err = partial(f);
  if (err != hipSuccess) return err;
  return merge(f);
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
