// Backward of the indexer over the kept keys: the gradient of the loss with respect to the
// kept keys' scores (the KL objective's dscores) carried into the indexer's own inputs.
// The twiscan post on GLM-5.2's IndexShare has the indexer trained to imitate the attention
// distribution through a KL loss; this is the chain rule of the Stage-1 score form
// ("GLM 5.2: How Four Co-Designed Mechanisms Beat Raw Scale", Part II, "DeepSeek Sparse
// Attention", Stage 1) score_j = sum_h w_h max(0, x_hj), x_hj = q_I[h,:] . k_I[s_j,:]:
//   dw_h    = sum_j g_j max(0, x_hj)
//   dq_I[h] = sum_j g_j w_h [x_hj > 0] k_I[s_j]
//   dk_I[s_j] += sum_h g_j w_h [x_hj > 0] q_I[h]
//
// One block per query, four waves; wave w owns indexer heads [16w, 16w + 16).  The block
// walks the query's kept keys in chunks of 32:
//  * the chunk's FP8 key rows are gathered into LDS twice: row-major (operands of the FP8
//    product) and dimension-major (operands of the dq product).  The gather runs ahead in
//    registers: the next chunk's rows, and the positions and d loss / d score one chunk
//    further, are loaded while a chunk is computed;
//  * each wave computes x^T for its heads with two FP8 MFMAs (A = key rows, B = its query
//    rows), so a lane holds four keys of one head: the layout of the A operand of the bf16
//    dq product over keys;
//  * the ReLU mask is decided exactly: where |x| from the MFMA is below 2^-10 |q_h| |k_j|,
//    the dot product is recomputed from the e4m3 bytes with fp32 products (exact: each is
//    an 8-bit significand) summed in fp64 (exact: at most 43 significant bits).  The FP8
//    MFMA's error has been measured at most 7.1e-5 |q| |k| (2.4e-4 of sum_c |q_c k_c|, on
//    codes spanning the whole e4m3 range), so the window holds it with a wide margin.  About
//    1 % of the dot products of random rows fall under the threshold;
//  * d loss / d x goes to LDS for all heads; the chunk's key gradients, summed over all
//    64 heads, are one bf16 product per 16x16 output tile (A = d loss / d x per key,
//    B = the query rows transposed), written to LDS and added to dk_I with row-contiguous
//    fp32 atomics (32 keys x d_I floats per chunk), or written as bf16 pair rows;
//  * d loss / d x enters the bf16 products as a hi + lo pair of bf16 (both rounded to
//    nearest: residual at most 2^-16 relative); the e4m3 operands are exact in bf16.
#include <algorithm>

#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

typedef float f32x2v __attribute__((ext_vector_type(2)));

constexpr int kBwdChunk = 32;
constexpr int kBwdThreads = 256;
constexpr int kBwdHeads = 64;
constexpr float kAmbiguous = 1.0f / 1024.0f;
// Waves per SIMD the register budget is cut for, per form.  The atomic form is bound by its
// atomics, and more waves only queue more of them.  The pair-row form is bound by its chunk
// latency, so it is cut to 168 VGPRs (a few spilled) for a third wave.
template <bool STORE>
constexpr int kBwdWaves = STORE ? 3 : 2;

typedef float f32x2v __attribute__((ext_vector_type(2)));

template <int DI>
struct __align__(16) BwdSmem {
  uint8_t q[kBwdHeads][DI];              // this query's rows; zero for heads >= H_I
  uint8_t krow[kBwdChunk][DI + 16];      // the chunk's key rows
  uint8_t kT[DI][kBwdChunk + 4];         // the same, dimension-major
  float g[kBwdChunk][kBwdHeads + 4];     // d loss / d x, [key][head]
  float dk[kBwdChunk][DI + 4];           // the chunk's key gradients
  float knorm[kBwdChunk];
  float ds[kBwdChunk];
  int32_t key[kBwdChunk];                // key position, or -1 for padding
};

template <bool HI>
__device__ __forceinline__ f32x2v e4m3_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

__device__ __forceinline__ float sumsq_e4m3(const uint32_t* w, int n_words) {
  float s = 0.f;
  for (int i = 0; i < n_words; ++i) {
    const f32x2v a = e4m3_pair<false>(w[i]), b = e4m3_pair<true>(w[i]);
    s = fmaf(a[0], a[0], s);
    s = fmaf(a[1], a[1], s);
    s = fmaf(b[0], b[0], s);
    s = fmaf(b[1], b[1], s);
  }
  return s;
}

// Exact dot product of two e4m3 rows of DI bytes (4-byte aligned).
template <int DI>
__device__ __forceinline__ float exact_dot_e4m3(const uint8_t* a, const uint8_t* b) {
  double acc = 0.0;
  for (int c = 0; c < DI; c += 4) {
    const uint32_t av = *reinterpret_cast<const uint32_t*>(a + c);
    const uint32_t bv = *reinterpret_cast<const uint32_t*>(b + c);
    const f32x2v a0 = e4m3_pair<false>(av), a1 = e4m3_pair<true>(av);
    const f32x2v b0 = e4m3_pair<false>(bv), b1 = e4m3_pair<true>(bv);
    acc += (double)(a0[0] * b0[0]);
    acc += (double)(a0[1] * b0[1]);
    acc += (double)(a1[0] * b1[0]);
    acc += (double)(a1[1] * b1[1]);
  }
  return (float)acc;
}

// Eight e4m3 bytes (lo: depth slots 0..3, hi: 4..7) -> bf16x8, exactly.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const f32x2v a = e4m3_pair<false>(lo), b = e4m3_pair<true>(lo);
  const f32x2v c = e4m3_pair<false>(hi), d = e4m3_pair<true>(hi);
  bf16x8 r;
  r[0] = (__bf16)a[0];
  r[1] = (__bf16)a[1];
  r[2] = (__bf16)b[0];
  r[3] = (__bf16)b[1];
  r[4] = (__bf16)c[0];
  r[5] = (__bf16)c[1];
  r[6] = (__bf16)d[0];
  r[7] = (__bf16)d[1];
  return r;
}

__device__ __forceinline__ __bf16 bf16_hi(float v) { return (__bf16)v; }
__device__ __forceinline__ __bf16 bf16_lo(float v, __bf16 hi) { return (__bf16)(v - (float)hi); }

// STORE: write each kept pair's dk_I row to `contrib` (bf16, or fp32 with F32ROWS) instead
// of adding it to dk.
template <int DI, bool STORE, bool F32ROWS = false>
__global__ __launch_bounds__(kBwdThreads, kBwdWaves<STORE>) void indexer_bwd_kernel(
    const uint8_t* __restrict__ qI, const uint8_t* __restrict__ kI, const float* __restrict__ w,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ idx,
    const float* __restrict__ dsc, int T, int S_max, int H, int k, float* __restrict__ dq,
    float* __restrict__ dw, float* __restrict__ dk, int64_t row0, void* __restrict__ contrib) {
  __shared__ BwdSmem<DI> sm;
  constexpr int kPieces = DI / 16;   // 16-byte pieces per row
  constexpr int kDimTiles = DI / 16;
  constexpr int kOwnTiles = DI / 32;  // dk output tiles of one wave (of 2 * DI / 16)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int64_t row = row0 + blockIdx.x;  // b * T + t
  const int b = (int)(row / T);
  int n_keys = kv_len[b];
  n_keys = n_keys < 0 ? 0 : (n_keys > S_max ? S_max : n_keys);
  const int32_t* idx_row = idx + row * k;
  const float* ds_row = dsc + row * k;

  // ---- the query's rows, and zero d loss / d x for heads that do not exist
  const uint8_t* qsrc = qI + row * H * DI;
  for (int i = tid; i < kBwdHeads * kPieces; i += kBwdThreads) {
    const int h = i / kPieces, p = i % kPieces;
    i32x4 v = {0, 0, 0, 0};
    if (h < H) v = ld_global_16(qsrc + h * DI + 16 * p);
    *reinterpret_cast<i32x4*>(&sm.q[h][16 * p]) = v;
  }
  for (int i = tid; i < kBwdChunk * (kBwdHeads + 4); i += kBwdThreads) (&sm.g[0][0])[i] = 0.f;
  __syncthreads();

  const int head = 16 * wv + l16;          // this lane's head in the x^T layout
  const bool wave_heads = 16 * wv < H;     // wave-uniform
  i32x8 qop = {0, 0, 0, 0, 0, 0, 0, 0};
  float qn = 0.f;
  if (32 * grp < DI) {
    qop = *reinterpret_cast<const i32x8*>(&sm.q[head][32 * grp]);
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(&sm.q[head][32 * grp]);
    qn = sumsq_e4m3(qw, 8);
  }
  qn += __shfl_xor(qn, 16);
  qn += __shfl_xor(qn, 32);
  qn = sqrtf(qn);
  const float w_h = head < H ? w[row * H + head] : 0.f;

  // B operands of the dk product: query rows transposed, depth = heads 32 ks + 8 grp + e
  const int kt_dk = wv & 1, ct0 = (wv >> 1) * kOwnTiles;
  bf16x8 qT[2][kOwnTiles];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int i = 0; i < kOwnTiles; ++i) {
      const int dim = 16 * (ct0 + i) + l16;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= (uint32_t)sm.q[32 * ks + 8 * grp + e][dim] << (8 * e);
        hi |= (uint32_t)sm.q[32 * ks + 8 * grp + 4 + e][dim] << (8 * e);
      }
      qT[ks][i] = e4m3x8_to_bf16(lo, hi);
    }
  }

  f32x4 dqacc[kDimTiles];
#pragma unroll
  for (int c = 0; c < kDimTiles; ++c) dqacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dwacc = 0.f;

  // The gather is pipelined through registers: thread (kk, p) holds piece p of kept key kk
  // of the next chunk, and the position and d loss / d score of that key one chunk further,
  // so their loads are in flight while a chunk is computed.  The position is checked only
  // where its piece is requested: checked at once, the wait for it would also wait for the
  // pieces requested just before it.
  const int kk = tid >> 3, p = tid & 7;
  auto load_sel = [&](int j, int& s, float& dsv) {  // as stored (-1, 0 past the row)
    s = -1;
    dsv = 0.f;
    if (j < k) {
      s = idx_row[j];
      dsv = ds_row[j];
    }
  };
  auto valid = [&](int s) { return s >= 0 && s < n_keys; };
  auto load_piece = [&](int s) {
    i32x4 v = {0, 0, 0, 0};
    if (valid(s) && p < kPieces) v = ld_global_16(kI + ((int64_t)b * S_max + s) * DI + 16 * p);
    return v;
  };
  int s_next, s_after;
  float ds_next, ds_after;
  load_sel(kk, s_next, ds_next);
  i32x4 v_next = load_piece(s_next);
  load_sel(kBwdChunk + kk, s_after, ds_after);

  for (int j0 = 0; j0 < k; j0 += kBwdChunk) {
    // ---- stage the chunk (piece p of kept key kk), then start loading the next two
    {
      const bool ok = valid(s_next);
      const int s = ok ? s_next : -1;
      const float dsv = ok ? ds_next : 0.f;
      const i32x4 v = v_next;
      const uint32_t vw[4] = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
      float ss = sumsq_e4m3(vw, 4);
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      if (p < kPieces) {
        *reinterpret_cast<i32x4*>(&sm.krow[kk][16 * p]) = v;
#pragma unroll
        for (int e = 0; e < 16; ++e) sm.kT[16 * p + e][kk] = (uint8_t)(vw[e >> 2] >> (8 * (e & 3)));
      }
      if (p == 0) {
        sm.knorm[kk] = sqrtf(ss);
        sm.ds[kk] = dsv;
        sm.key[kk] = s;
      }
      s_next = s_after;
      ds_next = ds_after;
      v_next = load_piece(s_next);
      load_sel(j0 + 2 * kBwdChunk + kk, s_after, ds_after);
      // nothing to add in this chunk (with a pair buffer every kept pair's row is written)
      if (!__syncthreads_or(s >= 0 && (STORE || dsv != 0.f))) continue;
    }

    // ---- x^T, the exact mask, d loss / d x, dw, and dq
    if (wave_heads) {
      f32x4 xt[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        i32x8 kop = {0, 0, 0, 0, 0, 0, 0, 0};
        if (32 * grp < DI) kop = *reinterpret_cast<const i32x8*>(&sm.krow[16 * kt + l16][32 * grp]);
        xt[kt] = mfma_e4m3_16x16x128(kop, qop);  // [key 16 kt + 4 grp + r][head l16]
      }
      // slot e = 4 kt + r holds key 16 kt + 4 grp + r
      float xs[8];
      uint32_t amb = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xs[e] = xt[e >> 2][e & 3];
        const int key = 16 * (e >> 2) + 4 * grp + (e & 3);
        if (fabsf(xs[e]) < kAmbiguous * qn * sm.knorm[key]) amb |= 1u << e;
      }
      while (amb) {  // rare: one exact recomputation per ambiguous entry
        const int e = __builtin_ctz(amb);
        amb &= amb - 1;
        const float ex = exact_dot_e4m3<DI>(&sm.q[head][0], &sm.krow[16 * (e >> 2) + 4 * grp + (e & 3)][0]);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (u == e) xs[u] = ex;
      }
      bf16x8 ghi, glo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * (e >> 2) + 4 * grp + (e & 3);
        const float dsk = sm.ds[key];
        dwacc = fmaf(dsk, fmaxf(xs[e], 0.f), dwacc);
        const float gv = xs[e] > 0.f ? dsk * w_h : 0.f;
        sm.g[key][head] = gv;
        const __bf16 h = bf16_hi(gv);
        ghi[e] = h;
        glo[e] = bf16_lo(gv, h);
      }
#pragma unroll
      for (int c = 0; c < kDimTiles; ++c) {
        const int dim = 16 * c + l16;
        const uint32_t lo = *reinterpret_cast<const uint32_t*>(&sm.kT[dim][4 * grp]);
        const uint32_t hi = *reinterpret_cast<const uint32_t*>(&sm.kT[dim][16 + 4 * grp]);
        const bf16x8 kb = e4m3x8_to_bf16(lo, hi);
        dqacc[c] = mfma_bf16_16x16x32(ghi, kb, dqacc[c]);  // [head 4 grp + r][dim l16]
        dqacc[c] = mfma_bf16_16x16x32(glo, kb, dqacc[c]);
      }
    }
    __syncthreads();

    // ---- the chunk's key gradients over all heads: wave tiles (kt_dk, ct0 .. ct0 + kOwnTiles)
    {
      f32x4 acc[kOwnTiles];
#pragma unroll
      for (int i = 0; i < kOwnTiles; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (32 * ks >= H) break;
        const float* gp = &sm.g[16 * kt_dk + l16][32 * ks + 8 * grp];
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gp + 4);
        bf16x8 ahi, alo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 h0 = bf16_hi(g0[e]), h1 = bf16_hi(g1[e]);
          ahi[e] = h0;
          alo[e] = bf16_lo(g0[e], h0);
          ahi[4 + e] = h1;
          alo[4 + e] = bf16_lo(g1[e], h1);
        }
#pragma unroll
        for (int i = 0; i < kOwnTiles; ++i) {
          acc[i] = mfma_bf16_16x16x32(ahi, qT[ks][i], acc[i]);  // [key 4 grp + r][dim l16]
          acc[i] = mfma_bf16_16x16x32(alo, qT[ks][i], acc[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kOwnTiles; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.dk[16 * kt_dk + 4 * grp + r][16 * (ct0 + i) + l16] = acc[i][r];
    }
    __syncthreads();

    // ---- with a pair buffer: the chunk's rows in bf16 or fp32, in pair order (summed per
    // key later), stored non-temporal (read back once, and too large to keep in the caches)
    if constexpr (STORE) {
      if constexpr (F32ROWS) {
        float* dst0 = reinterpret_cast<float*>(contrib) + ((size_t)(row - row0) * k + j0) * DI;
        for (int r = 8 * wv; r < 8 * wv + 8; ++r) {
          if (j0 + r >= k) break;
          if (2 * lane < DI)
            __builtin_nontemporal_store(
                (f32x2v){sm.dk[r][2 * lane], sm.dk[r][2 * lane + 1]},
                reinterpret_cast<f32x2v*>(dst0 + (size_t)r * DI + 2 * lane));
        }
        __syncthreads();
        continue;
      }
      uint16_t* dst0 = reinterpret_cast<uint16_t*>(contrib) + ((size_t)(row - row0) * k + j0) * DI;
      for (int r = 8 * wv; r < 8 * wv + 8; ++r) {
        if (j0 + r >= k) break;
        if (2 * lane < DI) {
          const uint32_t v = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)sm.dk[r][2 * lane]) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)sm.dk[r][2 * lane + 1]) << 16);
          __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(dst0 + (size_t)r * DI + 2 * lane));
        }
      }
      __syncthreads();
      continue;
    }
    // ---- add them to dk_I: wave w takes keys 8w .. 8w + 7, 64 consecutive floats per instruction
    for (int kk = 8 * wv; kk < 8 * wv + 8; ++kk) {
      const int s = sm.key[kk];
      if (s < 0 || sm.ds[kk] == 0.f) continue;
      float* dst = dk + ((int64_t)b * S_max + s) * DI;
#pragma unroll
      for (int c = lane; c < DI; c += 64) atomicAdd(dst + c, sm.dk[kk][c]);
    }
    __syncthreads();  // the next chunk overwrites the rows, keys and gradients
  }

  if (wave_heads) {
    dwacc += __shfl_xor(dwacc, 16);
    dwacc += __shfl_xor(dwacc, 32);
    if (grp == 0 && head < H) dw[row * H + head] = dwacc;
#pragma unroll
    for (int c = 0; c < kDimTiles; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * wv + 4 * grp + r;
        if (h < H) dq[(row * H + h) * DI + 16 * c + l16] = dqacc[c][r];
      }
  }
}

}  // namespace

hipError_t launch_indexer_bwd(const uint8_t* qI, const uint8_t* kI, const float* w,
                              const int32_t* kv_len, const int32_t* idx, const float* dscores,
                              int B, int T, int S_max, int H_I, int d_I, int k, float* dq,
                              float* dw, float* dk, bool f32_rows, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  auto grad = [&](int64_t row0, int64_t rows, void* contrib) {
    const dim3 grid((unsigned)rows), block(kBwdThreads);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, block, 0, stream, qI, kI, w, kv_len, idx, dscores, T, S_max,
                         H_I, k, dq, dw, dk, row0, contrib);
    };
    if (d_I == 128) {
      if (!contrib) go(indexer_bwd_kernel<128, false>);
      else if (f32_rows) go(indexer_bwd_kernel<128, true, true>);
      else go(indexer_bwd_kernel<128, true>);
    } else {
      if (!contrib) go(indexer_bwd_kernel<64, false>);
      else if (f32_rows) go(indexer_bwd_kernel<64, true, true>);
      else go(indexer_bwd_kernel<64, true>);
    }
  };
  const int64_t all = (int64_t)B * T;
  if (!ws) {
    grad(0, all, nullptr);
    return hipGetLastError();
  }
  // atomic-free: per pass, the inverted selection, pair rows of dk_I (bf16 or fp32), key sums
  const size_t row_bytes = (size_t)d_I * (f32_rows ? 4 : 2);
  const int64_t per_pass = pair_rows_per_pass(B, T, S_max, k, row_bytes, ws_bytes);
  if (per_pass < 1) return hipErrorInvalidValue;
  const PairLayout L = pair_layout(B, S_max, k, per_pass, row_bytes);
  void* contrib = reinterpret_cast<char*>(ws) + L.contrib;
  for (int64_t r0 = 0; r0 < all; r0 += per_pass) {
    const int64_t rows = std::min(per_pass, all - r0);
    hipError_t e = launch_pair_index(idx, kv_len, T, S_max, k, r0, rows, L, ws, stream);
    if (e != hipSuccess) return e;
    grad(r0, rows, contrib);
    e = launch_pair_reduce(L, ws, d_I, f32_rows, 1, dk, dk + d_I / 2, d_I, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ix
