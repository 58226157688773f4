// Sparse attention over the selected keys ("GLM 5.2: How Four Co-Designed Mechanisms
// Beat Raw Scale", Part II, "DeepSeek Sparse Attention", Stage 2: the kept tokens get
// full attention).  For each query token and KV head:
//   p = softmax_j(sm_scale * q_h . K[idx_j]),  out_h = sum_j p_j V[idx_j].
//
// Block = 4 waves on one (query token, KV head); the selection is cut into chunks
// of 32 entries and wave w takes chunks w, w+4, ...  Per chunk:
//  * gather: the chunk's 32 K rows and 32 V rows are fetched with 16-byte loads in
//    which consecutive lanes read consecutive pieces of one row (a whole row per
//    D/8 lanes), so every load touches only a few cache lines; rows are staged in
//    LDS with a bank swizzle.  The gathers of the wave's next two chunks are in
//    flight during a chunk's arithmetic (two register sets alternate).
//  * S^T = K Q^T (bf16 MFMA 16x16x32): K rows come from LDS as A operands; the (up
//    to 16) query heads that share the KV head are the columns, so lane (g, h) holds
//    keys {4g+i, 16+4g+i} of head h.
//  * online softmax in the exp2 domain, one running max per head; the max across the
//    four lane groups uses permlane swaps (no LDS round trip).
//  * O^T += V^T P^T: P^T is the B operand straight from the lanes that computed S^T;
//    V^T operands are read with the gfx950 transposing LDS read (each lane receives
//    four keys of one column), so output lane (g, h) holds head h and the per-head
//    rescale stays in-lane.
// The four waves' (m, l, O) are merged through LDS at the end.  Small batches split
// the selection over several blocks and merge the normalised partials by lse; when one
// layer's grid is that small, the layers of an IndexShare group share one launch (each
// block serves one layer and does exactly the work of the single-layer launch).
#include <algorithm>

#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

constexpr int kAttnWaves = 4;
constexpr int kAttnBlock = kAttnWaves * kWave;
constexpr int kChunk = 32;

// Layers whose attention one launch can run: each block serves one layer, with the same
// work and the same result as a launch for that layer alone.
constexpr int kAttnMaxLayers = 8;

struct AttnArgs {
  const uint16_t* q[kAttnMaxLayers];
  const uint16_t* kc[kAttnMaxLayers];
  const uint16_t* vc[kAttnMaxLayers];
  uint16_t* out[kAttnMaxLayers];
  float* lse[kAttnMaxLayers];
  float* part_o[kAttnMaxLayers];    // [rows * H_kv * n_splits][16][D] normalised partials
  float* part_lse[kAttnMaxLayers];  // [rows * H_kv * n_splits][16] natural-log partial lse
  const int32_t* idx;
  const int32_t* kv_len;
  int B, T, S_max, H_q, H_kv, grp, k;
  float scale_log2;  // sm_scale * log2(e)
  int n_splits, chunks, chunks_per_split;
  int layers;
  unsigned blocks_per_layer;
};

// Entry `layer` (wave-uniform) of a per-layer pointer array, picked with selects so the
// argument block is never copied to private memory.
template <typename T>
__device__ __forceinline__ T pick_layer(T const (&a)[kAttnMaxLayers], int layer) {
  T v = a[0];
#pragma unroll
  for (int l = 1; l < kAttnMaxLayers; ++l) v = layer == l ? a[l] : v;
  return v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, ld_global_16(p));
}

// Reductions across the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48).
// v_permlane16_swap x, y exchanges x's rows 1, 3 with y's rows 0, 2 (v_permlane32_swap:
// x's upper half with y's lower half).  With y a copy of x, x and y then hold each row
// and its neighbour, so one max/add per stage pairs the rows.  Written as asm with both
// registers read-write: the compiler's model of the builtin drops one of the two
// results when the operands are equal.  The s_nop's give the VALU <-> permlane hazard
// its wait states.
__device__ __forceinline__ void row_pair_swap16(uint32_t& x, uint32_t& y) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void row_pair_swap32(uint32_t& x, uint32_t& y) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ float max_across_rows(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  row_pair_swap16(x, y);
  v = fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
  x = y = __builtin_bit_cast(uint32_t, v);
  row_pair_swap32(x, y);
  return fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}
__device__ __forceinline__ float sum_across_rows(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  row_pair_swap16(x, y);
  v = __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
  x = y = __builtin_bit_cast(uint32_t, v);
  row_pair_swap32(x, y);
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}

// Transposing LDS read: within each 16-lane group, lane i receives element (i & 3) of
// the 8-byte reads of lanes 4r + (i >> 2), r = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// Bank swizzle of the staged K/V rows: 16-byte piece p of chunk slot n sits at piece
// position p ^ swz(n).  Rows are 256 B (D = 128: one row per 64-bank line) or 128 B
// (D = 64: two rows per line); swz rotates the slot's position within the line left by
// one bit, so the 16 slots of an A-operand read hit 16 distinct 16-byte bank groups and
// the 8 slots of a half-wave transposed read hit 8 distinct 32-byte groups.
template <int D>
__device__ __forceinline__ int stage_swz(int n) {
  constexpr int PI = D / 8;                     // 16-byte pieces per row
  constexpr int LOG = D == 128 ? 4 : 3;
  const int m = (D == 128 ? n : (n >> 1)) & (PI - 1);
  return ((m << 1) & (PI - 1)) | (m >> (LOG - 1));
}

// ML: the grid covers several layers (p.layers > 1); a single-layer launch reads entry 0
// of the pointer arrays directly.
template <int D, bool ML>
__global__ __launch_bounds__(kAttnBlock, 2) void sparse_attn_kernel(AttnArgs p) {
  constexpr int MC = D / 32;          // depth tiles of the QK^T product
  constexpr int NT = D / 16;          // 16-row tiles of O^T
  constexpr int ROWB = D * 2;         // bytes per K or V row
  constexpr int PI = ROWB / 16;       // 16-byte pieces per row
  constexpr int RPI = kWave / PI;     // rows per 64-lane load
  constexpr int NI = kChunk / RPI;    // loads per chunk per tensor
  __shared__ __attribute__((aligned(16))) unsigned char stage_all[kAttnWaves][2][kChunk * ROWB];
  __shared__ float ml_all[kAttnWaves][2][16];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  // XCD-aware order: the hardware deals consecutive blocks to the 8 XCDs in turn, so
  // block i runs on XCD i % 8; give each XCD a contiguous range of rows so nearby
  // queries (which tend to select overlapping keys) share one L2.
  unsigned bid = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
  const int layer = ML ? (int)(bid / p.blocks_per_layer) : 0;
  if (ML) bid -= (unsigned)layer * p.blocks_per_layer;
  const uint16_t* const q_l = pick_layer(p.q, layer);
  const uint16_t* const kc_l = pick_layer(p.kc, layer);
  const uint16_t* const vc_l = pick_layer(p.vc, layer);
  const int split = bid % p.n_splits;
  const int64_t rk = bid / p.n_splits;  // (b*T + t) * H_kv + kvh
  const int kvh = (int)(rk % p.H_kv);
  const int64_t row = rk / p.H_kv;      // b*T + t
  const int b = (int)(row / p.T);
  int kvl = p.kv_len ? p.kv_len[b] : p.S_max;
  kvl = kvl < 0 ? 0 : (kvl > p.S_max ? p.S_max : kvl);

  // Q as the B operand of S^T = K Q^T: column = head, depth slice [32m + 8lg, +8)
  bf16x8 qb[MC];
  const bool hvalid = r16 < p.grp;
  {
    const int head = kvh * p.grp + (hvalid ? r16 : 0);
    const uint16_t* qrow = q_l + ((size_t)row * p.H_q + head) * D;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      qb[m] = load_bf16x8(qrow + 32 * m + 8 * lg);
      if (!hvalid) qb[m] = (bf16x8){};
    }
  }

  const int32_t* irow = p.idx + (size_t)row * p.k;
  const uint32_t kv_stride_b = (uint32_t)(p.H_kv * ROWB);
  const size_t seq_off = ((size_t)b * p.S_max * p.H_kv + kvh) * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc_l + seq_off, (uint32_t)kvl * kv_stride_b);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc_l + seq_off, (uint32_t)kvl * kv_stride_b);
  unsigned char* kst = stage_all[wid][0];
  unsigned char* vst = stage_all[wid][1];

  // Gather layout: lane (rho = lane / PI, s = lane % PI) of load j fetches piece s of
  // chunk slot n = rho * NI + j, so each row is read by PI consecutive lanes.
  const int rho = lane / PI, s = lane % PI;
  uint32_t woff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int n = rho * NI + j;
    woff[j] = (uint32_t)(n * ROWB + 16 * (s ^ stage_swz<D>(n)));
  }
  // A operand of S^T (key tile tt = 0; tile 1 is 16 rows further): slot r16, piece 4m+lg
  uint32_t koff[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) koff[m] = (uint32_t)(r16 * ROWB + 16 * ((4 * m + lg) ^ stage_swz<D>(r16)));
  // transposed V read: slot 4lg + r16/4 (+16), logical bytes [32nt + 8(r16 & 3), +8)
  uint32_t voff[NT];
  {
    const int n = 4 * lg + (r16 >> 2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      voff[nt] = (uint32_t)(n * ROWB + 16 * ((2 * nt + ((r16 >> 1) & 1)) ^ stage_swz<D>(n)) + 8 * (r16 & 1));
  }

  float m_run = -__builtin_inff();  // running max of head r16 (log2 domain)
  float l_run = 0.f;                // this lane's share of the running sum
  f32x4 o[NT];                      // O^T: rows 16nt + 4lg + i (d), column r16 (head)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int c_begin = split * p.chunks_per_split;
  const int c_end = min(c_begin + p.chunks_per_split, p.chunks);
  const bool idx_vec = (p.k & 3) == 0;

  // Selected positions of this lane's NI slots of chunk c (-1: padding or not visible).
  auto load_idx = [&](int c, int (&jv)[NI]) {
    const int e0 = c * kChunk + rho * NI;
    if (c >= c_end) {
#pragma unroll
      for (int j = 0; j < NI; ++j) jv[j] = -1;
    } else if (idx_vec && c * kChunk + kChunk <= p.k) {
#pragma unroll
      for (int j = 0; j < NI; j += 4) {
        const i32x4 v = ld_global_16(irow + e0 + j);
        jv[j] = v[0]; jv[j + 1] = v[1]; jv[j + 2] = v[2]; jv[j + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) jv[j] = e0 + j < p.k ? irow[e0 + j] : -1;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) jv[j] = (jv[j] >= 0 && jv[j] < kvl) ? jv[j] : -1;
  };
  // Bit n of the result: slot n of the chunk holds a valid key.
  auto slot_mask = [&](const int (&jv)[NI]) -> uint32_t {
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) bits |= (jv[j] >= 0 ? 1u : 0u) << j;
    uint32_t mask = 0;
#pragma unroll
    for (int r = 0; r < RPI; ++r) mask |= (uint32_t)__builtin_amdgcn_readlane((int)bits, r * PI) << (r * NI);
    return mask;
  };
  // Two register sets of chunk rows alternate: while a chunk is computed, the gathers of
  // the next two chunks of this wave are in flight.
  i32x4 kdA[NI], vdA[NI], kdB[NI], vdB[NI];
  auto issue_rows = [&](const int (&jv)[NI], i32x4 (&kd)[NI], i32x4 (&vd)[NI]) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const uint32_t off = jv[j] >= 0 ? (uint32_t)jv[j] * kv_stride_b + 16u * s : 0x80000000u;
      kd[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
      vd[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, 0));
    }
  };

  constexpr int W = kAttnWaves;
  int jv[NI];  // positions of the next chunk to gather
  const int c0 = c_begin + wid;
  load_idx(c0, jv);
  uint32_t maskA = slot_mask(jv);
  issue_rows(jv, kdA, vdA);
  load_idx(c0 + W, jv);
  uint32_t maskB = slot_mask(jv);
  issue_rows(jv, kdB, vdB);
  load_idx(c0 + 2 * W, jv);

  // chunk c, whose rows are in (kd, vd): stage them (bank-swizzled), refill the set with
  // chunk c + 2W, then compute
  auto step = [&](int c, i32x4 (&kd)[NI], i32x4 (&vd)[NI], uint32_t& mask) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      *reinterpret_cast<i32x4*>(kst + woff[j]) = kd[j];
      *reinterpret_cast<i32x4*>(vst + woff[j]) = vd[j];
    }
    const uint32_t vmask = mask;
    if (c + 2 * W < c_end) {
      mask = slot_mask(jv);
      issue_rows(jv, kd, vd);
      load_idx(c + 3 * W, jv);
    }
    lds_wait();

    // S^T tiles: lane holds keys 16*tt + 4*lg + i for head r16
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(kst + koff[m]);
      const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(kst + koff[m] + 16 * ROWB);
      s0 = mfma_bf16_16x16x32(ka0, qb[m], s0);
      s1 = mfma_bf16_16x16x32(ka1, qb[m], s1);
    }
    float x[8];
    float mloc = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok0 = (vmask >> (4 * lg + i)) & 1u;
      const bool ok1 = (vmask >> (16 + 4 * lg + i)) & 1u;
      x[i] = ok0 ? s0[i] * p.scale_log2 : -__builtin_inff();
      x[4 + i] = ok1 ? s1[i] * p.scale_log2 : -__builtin_inff();
      mloc = fmaxf(mloc, fmaxf(x[i], x[4 + i]));
    }
    mloc = max_across_rows(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const bool any = m_new != -__builtin_inff();
    const float alpha = (any && m_run != -__builtin_inff()) ? exp2f(m_run - m_new) : (any ? 0.f : 1.f);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = (x[e] != -__builtin_inff()) ? exp2f(x[e] - m_new) : 0.f;
      psum += pr[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nt][i] *= alpha;

    // P^T as the B operand: column = head r16, depth slots = keys
    // {4lg..4lg+3, 16+4lg..16+4lg+3}
    bf16x8 pb;
    {
      i32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pk[e] = (int)((uint32_t)f32_to_bf16_rne(pr[2 * e]) |
                      ((uint32_t)f32_to_bf16_rne(pr[2 * e + 1]) << 16));
      pb = __builtin_bit_cast(bf16x8, pk);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // V^T rows 16nt..16nt+15 (d), depth = the same 8 keys as P^T
      const i16x4 lo = lds_read_tr16(vst + voff[nt]);
      const i16x4 hi = lds_read_tr16(vst + voff[nt] + 16 * ROWB);
      const bf16x8 va = __builtin_bit_cast(
          bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      o[nt] = mfma_bf16_16x16x32(va, pb, o[nt]);
    }
    lds_wait();
  };
  for (int c = c0; c < c_end; c += 2 * W) {
    step(c, kdA, vdA, maskA);
    if (c + W < c_end) step(c + W, kdB, vdB, maskB);
  }

  // per-head l: sum the four lane groups' shares
  l_run = sum_across_rows(l_run);

  // merge the 4 waves through LDS: os[head][d]
  __syncthreads();
  float* os = reinterpret_cast<float*>(kst);
  static_assert(16 * D * sizeof(float) <= 2 * kChunk * ROWB, "O staging");
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) os[r16 * D + 16 * nt + 4 * lg + i] = o[nt][i];
  if (lg == 0) {
    ml_all[wid][0][r16] = m_run;
    ml_all[wid][1][r16] = l_run;
  }
  __syncthreads();

  const float ln2 = 0.69314718055994530942f;
  for (int e = threadIdx.x; e < 16 * D; e += kAttnBlock) {
    const int h = e / D, dcol = e % D;
    if (h >= p.grp) continue;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml_all[w][0][h]);
    float L = 0.f, acc = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = ml_all[w][0][h];
        const float f = mw == -__builtin_inff() ? 0.f : exp2f(mw - M);
        L += f * ml_all[w][1][h];
        acc += f * reinterpret_cast<const float*>(stage_all[w][0])[h * D + dcol];
      }
    }
    const float val = L > 0.f ? acc / L : 0.f;
    const float lse_v = L > 0.f ? (M + log2f(L)) * ln2 : -__builtin_inff();
    const int head = kvh * p.grp + h;
    if (p.n_splits == 1) {
      pick_layer(p.out, layer)[((size_t)row * p.H_q + head) * D + dcol] = f32_to_bf16_rne(val);
      float* const lse_l = pick_layer(p.lse, layer);
      if (lse_l && dcol == 0) lse_l[(size_t)row * p.H_q + head] = lse_v;
    } else {
      const size_t pr = (size_t)rk * p.n_splits + split;
      pick_layer(p.part_o, layer)[(pr * 16 + h) * D + dcol] = val;
      if (dcol == 0) pick_layer(p.part_lse, layer)[pr * 16 + h] = lse_v;
    }
  }
}

// Merge of split partials: out = sum_s exp(lse_s - LSE) o_s, LSE = log sum_s exp(lse_s).
// One thread per output element (row, KV head, head of the group, column).
template <int D>
__global__ __launch_bounds__(256) void sparse_attn_combine_kernel(AttnArgs p, int64_t per_layer) {
  int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= per_layer * p.layers) return;
  const int layer = (int)(gid / per_layer);
  gid -= layer * per_layer;
  const int dcol = (int)(gid % D);
  const int64_t rh = gid / D;
  const int h = (int)(rh % p.grp);
  const int64_t rk = rh / p.grp;  // row * H_kv + kvh
  const int kvh = (int)(rk % p.H_kv);
  const int64_t row = rk / p.H_kv;
  const float* lse_p = pick_layer(p.part_lse, layer) + (size_t)rk * p.n_splits * 16 + h;
  const float* o_p = pick_layer(p.part_o, layer) + ((size_t)rk * p.n_splits * 16 + h) * D + dcol;
  float M = -__builtin_inff();
  for (int s = 0; s < p.n_splits; ++s) M = fmaxf(M, lse_p[s * 16]);
  float acc = 0.f, L = 0.f;
  if (M != -__builtin_inff()) {
#pragma unroll 4
    for (int s = 0; s < p.n_splits; ++s) {
      const float ls = lse_p[s * 16];
      const float f = ls == -__builtin_inff() ? 0.f : __expf(ls - M);
      L += f;
      acc += f * o_p[(size_t)s * 16 * D];
    }
  }
  const int head = kvh * p.grp + h;
  pick_layer(p.out, layer)[((size_t)row * p.H_q + head) * D + dcol] =
      f32_to_bf16_rne(L > 0.f ? acc / L : 0.f);
  float* const lse_l = pick_layer(p.lse, layer);
  if (lse_l && dcol == 0)
    lse_l[(size_t)row * p.H_q + head] = L > 0.f ? M + __logf(L) : -__builtin_inff();
}

// ------------------------------------------------------------------ backward

struct AttnBwdArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* idx;
  const int32_t* kv_len;
  const uint16_t* out;
  const float* lse;
  const uint16_t* dout;
  int B, T, S_max, H_q, H_kv, grp, k, chunks;
  float scale;       // sm_scale
  float scale_log2;  // sm_scale * log2(e)
  float* dq;
  float* dkc;
  float* dvc;
  int64_t row0;       // first query row (b * T + t) of this launch
  uint16_t* contrib;  // non-null: per-pair dV | dK rows (bf16) instead of atomics
};

// bf16 16x16x16: D += A(16x16) * B(16x16); lane l supplies A[l & 15][4(l>>4) .. +3] and
// B[4(l>>4) .. +3][l & 15].
__device__ __forceinline__ f32x4 mfma_bf16_16x16x16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// Gradients of the sparse attention (the training side named by the twiscan post: the
// indexer learns from the attention distribution; these are the attention's own
// gradients over the selected rows).  With p = softmax(sm_scale q K_J^T) per head,
// D = dO . O:  dV_j += p_j dO,  dS_j = p_j (dO . V_j - D),  dq = sm_scale sum_j dS_j K_j,
// dK_j += sm_scale dS_j q.
// Block = 4 waves on one (query token, KV head), wave w taking chunks w, w+4, ... of 32
// selected rows, gathered into LDS exactly as in the forward kernel.  Per chunk:
//  * S^T = K Q^T and dP^T = V dO^T (bf16 MFMA 16x16x32, K and V rows from LDS as A
//    operands, heads as columns); P and dS are formed in the lanes that hold them, with
//    the forward's lse;
//  * dq^T += K^T dS^T, as the forward's O^T += V^T P^T (transposing LDS reads of K);
//  * P and sm_scale * dS go to a small LDS tile [head][key] and come back through the
//    transposing read as the A operands (keys x heads) of 16x16x16 products with Q and dO
//    (heads x d), giving dV and dK rows that are added to the fp32 gradient caches with
//    float atomics (the same key is selected by many queries).
// The four waves' dq^T partials are summed through LDS.
template <int D>
__global__ __launch_bounds__(kAttnBlock, 2) void sparse_attn_bwd_kernel(AttnBwdArgs p) {
  constexpr int MC = D / 32;
  constexpr int NT = D / 16;
  constexpr int ROWB = D * 2;
  constexpr int PI = ROWB / 16;
  constexpr int RPI = kWave / PI;
  constexpr int NI = kChunk / RPI;
  constexpr int PROW = kChunk + 4;  // bf16 per row of a P / dS tile (4 of padding)
  __shared__ __attribute__((aligned(16))) unsigned char stage_all[kAttnWaves][2][kChunk * ROWB];
  __shared__ __attribute__((aligned(16))) uint16_t pt_all[kAttnWaves][2][16 * PROW];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  unsigned bid = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
  const int64_t rk = bid + p.row0 * p.H_kv;  // (b*T + t) * H_kv + kvh
  const int kvh = (int)(rk % p.H_kv);
  const int64_t row = rk / p.H_kv;
  const int b = (int)(row / p.T);
  int kvl = p.kv_len ? p.kv_len[b] : p.S_max;
  kvl = kvl < 0 ? 0 : (kvl > p.S_max ? p.S_max : kvl);

  // this lane's head r16: q and dO as B operands [head][32m + 8lg, +8), D = dO . O, lse
  const bool hvalid = r16 < p.grp;
  const int head = kvh * p.grp + (hvalid ? r16 : 0);
  const size_t hrow = ((size_t)row * p.H_q + head) * D;
  bf16x8 qb[MC], dob[MC];
  float dpart = 0.f;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    qb[m] = load_bf16x8(p.q + hrow + 32 * m + 8 * lg);
    dob[m] = load_bf16x8(p.dout + hrow + 32 * m + 8 * lg);
    const i32x4 ov = ld_global_16(p.out + hrow + 32 * m + 8 * lg);
    const i32x4 dv = __builtin_bit_cast(i32x4, dob[m]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t o2 = (uint32_t)ov[e], d2 = (uint32_t)dv[e];
      dpart = fmaf(bf16_to_f32((uint16_t)o2), bf16_to_f32((uint16_t)d2), dpart);
      dpart = fmaf(bf16_to_f32((uint16_t)(o2 >> 16)), bf16_to_f32((uint16_t)(d2 >> 16)), dpart);
    }
    if (!hvalid) {
      qb[m] = (bf16x8){};
      dob[m] = (bf16x8){};
    }
  }
  const float Dh = hvalid ? sum_across_rows(dpart) : 0.f;
  const float lse_h = hvalid ? p.lse[(size_t)row * p.H_q + head] : -__builtin_inff();
  const float lse2 = lse_h == -__builtin_inff() ? __builtin_inff() : lse_h * 1.4426950408889634f;

  // q and dO as B operands of the 16x16x16 products: rows (heads) 4lg..4lg+3, column
  // 16nt + r16
  i16x4 qB[NT], doB[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h2 = 4 * lg + i;
      const size_t off = ((size_t)row * p.H_q + kvh * p.grp + h2) * D + 16 * nt + r16;
      qB[nt][i] = h2 < p.grp ? (short)p.q[off] : (short)0;
      doB[nt][i] = h2 < p.grp ? (short)p.dout[off] : (short)0;
    }
  }

  const int32_t* irow = p.idx + (size_t)row * p.k;
  const uint32_t kv_stride_b = (uint32_t)(p.H_kv * ROWB);
  const size_t seq_off = ((size_t)b * p.S_max * p.H_kv + kvh) * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.kc + seq_off, (uint32_t)kvl * kv_stride_b);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.vc + seq_off, (uint32_t)kvl * kv_stride_b);
  float* dk_seq = p.dkc + seq_off;
  float* dv_seq = p.dvc + seq_off;
  unsigned char* kst = stage_all[wid][0];
  unsigned char* vst = stage_all[wid][1];
  uint16_t* ptp = pt_all[wid][0];
  uint16_t* pts = pt_all[wid][1];

  const int rho = lane / PI, s = lane % PI;
  uint32_t woff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int n = rho * NI + j;
    woff[j] = (uint32_t)(n * ROWB + 16 * (s ^ stage_swz<D>(n)));
  }
  uint32_t koff[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) koff[m] = (uint32_t)(r16 * ROWB + 16 * ((4 * m + lg) ^ stage_swz<D>(r16)));
  uint32_t toff[NT];  // transposed reads of the staged K rows (as V in the forward)
  {
    const int n = 4 * lg + (r16 >> 2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      toff[nt] = (uint32_t)(n * ROWB + 16 * ((2 * nt + ((r16 >> 1) & 1)) ^ stage_swz<D>(n)) + 8 * (r16 & 1));
  }
  // P / dS tiles: written as rows [head][key] by the lanes that hold them, read
  // transposed: lane (lg, r16) reads row 4lg + r16/4, keys 4(r16 & 3) .. +3 of a half
  const int pt_w = r16 * PROW + 4 * lg;
  const int pt_r = (4 * lg + (r16 >> 2)) * PROW + 4 * (r16 & 3);

  f32x4 dqa[NT];  // dq^T: rows 16nt + 4lg + i (d), column r16 (head)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) dqa[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int c_end = p.chunks;
  const bool idx_vec = (p.k & 3) == 0;
  auto load_idx = [&](int c, int (&jv)[NI]) {
    const int e0 = c * kChunk + rho * NI;
    if (c >= c_end) {
#pragma unroll
      for (int j = 0; j < NI; ++j) jv[j] = -1;
    } else if (idx_vec && c * kChunk + kChunk <= p.k) {
#pragma unroll
      for (int j = 0; j < NI; j += 4) {
        const i32x4 v = ld_global_16(irow + e0 + j);
        jv[j] = v[0]; jv[j + 1] = v[1]; jv[j + 2] = v[2]; jv[j + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) jv[j] = e0 + j < p.k ? irow[e0 + j] : -1;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) jv[j] = (jv[j] >= 0 && jv[j] < kvl) ? jv[j] : -1;
  };
  i32x4 kd[NI], vd[NI];
  auto issue_rows = [&](const int (&jv)[NI]) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const uint32_t off = jv[j] >= 0 ? (uint32_t)jv[j] * kv_stride_b + 16u * s : 0x80000000u;
      kd[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
      vd[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, 0));
    }
  };
  // cache rows of the keys this lane's S^T values belong to: keys 16tt + 4lg + i
  auto key_rows = [&](int c, int (&kr)[8]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = c * kChunk + 16 * tt + 4 * lg + i;
        int j = e < p.k ? irow[e] : -1;
        kr[4 * tt + i] = (j >= 0 && j < kvl) ? j : -1;
      }
  };

  // (no cross-chunk prefetch here: the registers go to the gradient operands instead)
  for (int c = wid; c < c_end; c += kAttnWaves) {
    int jv[NI];
    load_idx(c, jv);
    issue_rows(jv);
    int kr[8];
    key_rows(c, kr);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      *reinterpret_cast<i32x4*>(kst + woff[j]) = kd[j];
      *reinterpret_cast<i32x4*>(vst + woff[j]) = vd[j];
    }
    lds_wait();

    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, dp0 = s0, dp1 = s0;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(kst + koff[m]);
      const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(kst + koff[m] + 16 * ROWB);
      const bf16x8 va0 = *reinterpret_cast<const bf16x8*>(vst + koff[m]);
      const bf16x8 va1 = *reinterpret_cast<const bf16x8*>(vst + koff[m] + 16 * ROWB);
      s0 = mfma_bf16_16x16x32(ka0, qb[m], s0);
      s1 = mfma_bf16_16x16x32(ka1, qb[m], s1);
      dp0 = mfma_bf16_16x16x32(va0, dob[m], dp0);
      dp1 = mfma_bf16_16x16x32(va1, dob[m], dp1);
    }
    float pr[8], ds[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok0 = kr[i] >= 0, ok1 = kr[4 + i] >= 0;
      pr[i] = ok0 ? exp2f(s0[i] * p.scale_log2 - lse2) : 0.f;
      pr[4 + i] = ok1 ? exp2f(s1[i] * p.scale_log2 - lse2) : 0.f;
      ds[i] = pr[i] * (dp0[i] - Dh);
      ds[4 + i] = pr[4 + i] * (dp1[i] - Dh);
    }

    // dq^T += K^T dS^T: dS^T as the B operand (column = head r16)
    {
      i32x4 dk;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dk[e] = (int)((uint32_t)f32_to_bf16_rne(ds[2 * e]) |
                      ((uint32_t)f32_to_bf16_rne(ds[2 * e + 1]) << 16));
      const bf16x8 dsb = __builtin_bit_cast(bf16x8, dk);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const i16x4 lo = lds_read_tr16(kst + toff[nt]);
        const i16x4 hi = lds_read_tr16(kst + toff[nt] + 16 * ROWB);
        const bf16x8 ka = __builtin_bit_cast(
            bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        dqa[nt] = mfma_bf16_16x16x32(ka, dsb, dqa[nt]);
      }
    }

    // P and sm_scale * dS as [head][key] tiles
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      i16x4 pv, sv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = (short)f32_to_bf16_rne(pr[4 * tt + i]);
        sv[i] = (short)f32_to_bf16_rne(ds[4 * tt + i] * p.scale);
      }
      *reinterpret_cast<i16x4*>(ptp + pt_w + 16 * tt) = pv;
      *reinterpret_cast<i16x4*>(pts + pt_w + 16 * tt) = sv;
    }
    lds_wait();

    // dV += P^T dO and dK += (sm_scale dS)^T Q, row by row into the gradient caches, or
    // (with a pair buffer) each selected pair's dV | dK rows in bf16, staged in the K / V
    // stage (no longer read in this chunk) and written in pair order
    if (p.contrib) {
      uint16_t* cb = reinterpret_cast<uint16_t*>(stage_all[wid][0]);
      static_assert(kChunk * 4 * D <= 2 * kChunk * ROWB, "pair staging");
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const i16x4 pa = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(ptp + pt_r + 16 * tt));
        const i16x4 sa = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(pts + pt_r + 16 * tt));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const f32x4 dv = mfma_bf16_16x16x16(pa, doB[nt], z);
          const f32x4 dk = mfma_bf16_16x16x16(sa, qB[nt], z);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 16 * tt + 4 * lg + i;
            cb[(2 * e) * D + 16 * nt + r16] = f32_to_bf16_rne(dv[i]);
            cb[(2 * e + 1) * D + 16 * nt + r16] = f32_to_bf16_rne(dk[i]);
          }
        }
      }
      lds_wait();
      constexpr int kPieces = 4 * D / 16;  // 16-byte pieces of one pair's dV | dK rows
      uint16_t* dst0 = p.contrib + ((size_t)(row - p.row0) * p.k * p.H_kv + kvh) * 2 * D;
      for (int q2 = lane; q2 < kChunk * kPieces; q2 += kWave) {
        const int e = q2 / kPieces, pc = q2 % kPieces;
        const int ent = c * kChunk + e;
        if (ent < p.k) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(cb + (size_t)e * 2 * D + 8 * pc);
          *reinterpret_cast<i32x4*>(dst0 + (size_t)ent * p.H_kv * 2 * D + 8 * pc) = v;
        }
      }
      lds_wait();
      continue;
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const i16x4 pa = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(ptp + pt_r + 16 * tt));
      const i16x4 sa = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(pts + pt_r + 16 * tt));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 dv = mfma_bf16_16x16x16(pa, doB[nt], z);
        const f32x4 dk = mfma_bf16_16x16x16(sa, qB[nt], z);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kr[4 * tt + i];
          if (j >= 0) {
            const size_t off = (size_t)j * p.H_kv * D + 16 * nt + r16;
            atomicAdd(dv_seq + off, dv[i]);
            atomicAdd(dk_seq + off, dk[i]);
          }
        }
      }
    }
    lds_wait();
  }

  // sum the four waves' dq^T partials through LDS: qs[head][d]
  __syncthreads();
  float* qs = reinterpret_cast<float*>(kst);
  static_assert(16 * D * sizeof(float) <= 2 * kChunk * ROWB, "dq staging");
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) qs[r16 * D + 16 * nt + 4 * lg + i] = dqa[nt][i];
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * D; e += kAttnBlock) {
    const int h = e / D, dcol = e % D;
    if (h >= p.grp) continue;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) acc += reinterpret_cast<const float*>(stage_all[w][0])[h * D + dcol];
    p.dq[((size_t)row * p.H_q + kvh * p.grp + h) * D + dcol] = acc * p.scale;
  }
}


// ------------------------------------------------------------------ indexer KL objective

// Training side of the indexer (the twiscan post on GLM-5.2's IndexShare: the indexer
// learns to imitate the attention distribution through a KL loss).  Per query, over the
// valid entries j of its selection:
//   u_j = sum_h exp(sm_scale q_h.K_j - lse_h)   (all H_q heads, lse from the forward)
//   t = u / sum_j u_j,  pred = softmax_j(score_j),
//   loss = sum_j t_j (log t_j - log pred_j),  dscore_j = pred_j - t_j.
// Block = 4 waves on one query; wave w takes chunks w, w+4, ... of 32 entries, gathers
// their K rows as the forward does and forms S = Q K^T with the heads as rows (lane
// (g, key) holds heads 4g+i), so the head sum is four in-lane adds and two permlane
// stages.  u goes to LDS; the block then reduces sum(u) and the scores' (max, sum exp)
// and writes the per-entry gradient and the loss.
struct KlArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const int32_t* idx;
  const int32_t* kv_len;
  const float* lse;  // [B*T][H_q] natural log
  const float* sc;   // [B*T][k] indexer scores of the entries
  int B, T, S_max, H_q, H_kv, grp, k, chunks;
  float scale_log2;  // sm_scale * log2(e)
  float* loss;       // [B*T]
  float* dsc;        // [B*T][k]
};

constexpr int kKlMaxK = 2048;  // the largest k the library accepts

// (max, sum exp(x - max)) pairs: combine without touching exp(-inf - -inf).
__device__ __forceinline__ void lse_combine(float& m, float& z, float m2, float z2) {
  if (m2 == -__builtin_inff()) return;
  if (m == -__builtin_inff()) { m = m2; z = z2; return; }
  if (m2 > m) { z = z * expf(m - m2) + z2; m = m2; }
  else z += z2 * expf(m2 - m);
}

template <int D>
__global__ __launch_bounds__(kAttnBlock, 2) void indexer_kl_kernel(KlArgs p) {
  constexpr int MC = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int PI = ROWB / 16;
  constexpr int RPI = kWave / PI;
  constexpr int NI = kChunk / RPI;
  __shared__ __attribute__((aligned(16))) unsigned char stage_all[kAttnWaves][kChunk * ROWB];
  __shared__ float ubuf[kKlMaxK];
  __shared__ float red[kAttnWaves][3];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  unsigned bid = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
  const int64_t row = bid;  // b*T + t
  const int b = (int)(row / p.T);
  int kvl = p.kv_len ? p.kv_len[b] : p.S_max;
  kvl = kvl < 0 ? 0 : (kvl > p.S_max ? p.S_max : kvl);

  const int32_t* irow = p.idx + (size_t)row * p.k;
  const uint32_t kv_stride_b = (uint32_t)(p.H_kv * ROWB);
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(p.kc + (size_t)b * p.S_max * p.H_kv * D, (uint32_t)kvl * kv_stride_b);
  unsigned char* kst = stage_all[wid];

  const int rho = lane / PI, s = lane % PI;
  uint32_t woff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int n = rho * NI + j;
    woff[j] = (uint32_t)(n * ROWB + 16 * (s ^ stage_swz<D>(n)));
  }
  // B operand of S = Q K^T: column = key slot r16 (+16 for the second tile), depth piece 4m+lg
  uint32_t koff[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) koff[m] = (uint32_t)(r16 * ROWB + 16 * ((4 * m + lg) ^ stage_swz<D>(r16)));

  // Q rows (A operand: row = head r16 of the group, depth [32m + 8lg, +8)) and the
  // log2-domain normalisers of heads 4lg+i (+inf for heads past the group: weight 0).
  const bool hvalid = r16 < p.grp;
  bf16x8 qa[MC];
  float lse2[4];
  auto load_head_data = [&](int kvh) {
    const uint16_t* qrow = p.q + ((size_t)row * p.H_q + kvh * p.grp + (hvalid ? r16 : 0)) * D;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      qa[m] = load_bf16x8(qrow + 32 * m + 8 * lg);
      if (!hvalid) qa[m] = (bf16x8){};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * lg + i;
      lse2[i] = h < p.grp ? p.lse[(size_t)row * p.H_q + kvh * p.grp + h] * 1.4426950408889634f
                          : __builtin_inff();
    }
  };

  const bool idx_vec = (p.k & 3) == 0;
  auto load_idx = [&](int c, int (&jv)[NI]) {
    const int e0 = c * kChunk + rho * NI;
    if (c >= p.chunks) {
#pragma unroll
      for (int j = 0; j < NI; ++j) jv[j] = -1;
    } else if (idx_vec && c * kChunk + kChunk <= p.k) {
#pragma unroll
      for (int j = 0; j < NI; j += 4) {
        const i32x4 v = ld_global_16(irow + e0 + j);
        jv[j] = v[0]; jv[j + 1] = v[1]; jv[j + 2] = v[2]; jv[j + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) jv[j] = e0 + j < p.k ? irow[e0 + j] : -1;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) jv[j] = (jv[j] >= 0 && jv[j] < kvl) ? jv[j] : -1;
  };
  auto slot_mask = [&](const int (&jv)[NI]) -> uint32_t {
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) bits |= (jv[j] >= 0 ? 1u : 0u) << j;
    uint32_t mask = 0;
#pragma unroll
    for (int r = 0; r < RPI; ++r) mask |= (uint32_t)__builtin_amdgcn_readlane((int)bits, r * PI) << (r * NI);
    return mask;
  };
  i32x4 kd[NI];
  auto issue_rows = [&](const int (&jv)[NI], int kvh) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const uint32_t off = jv[j] >= 0 ? (uint32_t)jv[j] * kv_stride_b + (uint32_t)(kvh * ROWB) + 16u * s
                                      : 0x80000000u;
      kd[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
    }
  };

  load_head_data(0);
  int jc[NI], jn[NI];
  const int c0 = wid;
  load_idx(c0, jc);
  uint32_t mask_c = slot_mask(jc);
  issue_rows(jc, 0);
  load_idx(c0 + kAttnWaves, jn);

  for (int c = c0; c < p.chunks; c += kAttnWaves) {
    const uint32_t vmask = mask_c;
    float u0 = 0.f, u1 = 0.f;  // this lane's heads, keys r16 and 16 + r16
    for (int kvh = 0; kvh < p.H_kv; ++kvh) {
#pragma unroll
      for (int j = 0; j < NI; ++j) *reinterpret_cast<i32x4*>(kst + woff[j]) = kd[j];
      if (kvh + 1 < p.H_kv) {
        issue_rows(jc, kvh + 1);
      } else if (c + kAttnWaves < p.chunks) {
        mask_c = slot_mask(jn);
        issue_rows(jn, 0);
#pragma unroll
        for (int j = 0; j < NI; ++j) jc[j] = jn[j];
        load_idx(c + 2 * kAttnWaves, jn);
      }
      if (p.H_kv > 1) load_head_data(kvh);  // one KV head: loaded once above
      lds_wait();
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < MC; ++m) {
        const bf16x8 kb0 = *reinterpret_cast<const bf16x8*>(kst + koff[m]);
        const bf16x8 kb1 = *reinterpret_cast<const bf16x8*>(kst + koff[m] + 16 * ROWB);
        s0 = mfma_bf16_16x16x32(qa[m], kb0, s0);
        s1 = mfma_bf16_16x16x32(qa[m], kb1, s1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u0 += exp2f(s0[i] * p.scale_log2 - lse2[i]);
        u1 += exp2f(s1[i] * p.scale_log2 - lse2[i]);
      }
      lds_wait();
    }
    u0 = sum_across_rows(u0);
    u1 = sum_across_rows(u1);
    if (lg == 0) {
      ubuf[c * kChunk + r16] = ((vmask >> r16) & 1u) ? u0 : 0.f;
      ubuf[c * kChunk + 16 + r16] = ((vmask >> (16 + r16)) & 1u) ? u1 : 0.f;
    }
  }
  __syncthreads();

  // block reductions: sum(u), and (max, sum exp) of the valid entries' scores
  const float* srow = p.sc + (size_t)row * p.k;
  float U = 0.f, m = -__builtin_inff(), z = 0.f;
  for (int j = threadIdx.x; j < p.k; j += kAttnBlock) {
    const int e = irow[j];
    if (e < 0 || e >= kvl) continue;
    U += ubuf[j];
    lse_combine(m, z, srow[j], 1.f);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    U += __shfl_xor(U, off);
    const float m2 = __shfl_xor(m, off), z2 = __shfl_xor(z, off);
    lse_combine(m, z, m2, z2);
  }
  if (lane == 0) {
    red[wid][0] = U;
    red[wid][1] = m;
    red[wid][2] = z;
  }
  __syncthreads();
  U = red[0][0];
  m = red[0][1];
  z = red[0][2];
#pragma unroll
  for (int w = 1; w < kAttnWaves; ++w) {
    U += red[w][0];
    lse_combine(m, z, red[w][1], red[w][2]);
  }
  const float log_z = m + logf(z);
  const float inv_u = U > 0.f ? 1.f / U : 0.f;
  float lsum = 0.f;
  float* drow = p.dsc + (size_t)row * p.k;
  for (int j = threadIdx.x; j < p.k; j += kAttnBlock) {
    const int e = irow[j];
    float g = 0.f;
    if (e >= 0 && e < kvl) {
      const float t = ubuf[j] * inv_u;
      const float lp = srow[j] - log_z;
      g = expf(lp) - t;
      if (t > 0.f) lsum += t * (logf(t) - lp);
    }
    drow[j] = g;
  }
  for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
  __syncthreads();
  if (lane == 0) red[wid][0] = lsum;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) tot += red[w][0];
    p.loss[row] = tot;
  }
}

}  // namespace

AttnPlan make_attn_plan(int B, int T, int H_q, int H_kv, int d, int k) {
  (void)H_q;
  AttnPlan p{};
  p.chunks = (k + kChunk - 1) / kChunk;
  const int64_t base = (int64_t)B * T * H_kv;
  int ns = 1;
  if (base > 0 && base < 1024) {
    // one round of resident blocks (2 per CU), at least two chunks per wave so the
    // gathers of a wave's next chunk overlap the current one
    const int64_t want = (512 + base - 1) / base;
    int64_t by_chunks = p.chunks / (2 * kAttnWaves);
    if (by_chunks < 1) by_chunks = 1;
    ns = (int)(want < by_chunks ? want : by_chunks);
  }
  p.n_splits = ns;
  p.chunks_per_split = (p.chunks + ns - 1) / ns;
  if (ns > 1) {
    const size_t parts = (size_t)base * ns;
    const size_t o_bytes = parts * 16 * d * sizeof(float);
    const size_t l_bytes = parts * 16 * sizeof(float);
    p.ws_bytes = ((o_bytes + 255) / 256) * 256 + ((l_bytes + 255) / 256) * 256;
  }
  return p;
}

hipError_t launch_sparse_attn_layers(int n_layers, const void* const* q, const void* const* kc,
                                     const void* const* vc, const int32_t* idx,
                                     const int32_t* kv_len, int B, int T, int S_max, int H_q,
                                     int H_kv, int d, int k, float sm_scale, void* const* out,
                                     float* const* lse, const AttnPlan& pl, void* ws,
                                     hipStream_t stream) {
  AttnArgs x{};
  x.idx = idx;
  x.kv_len = kv_len;
  x.B = B;
  x.T = T;
  x.S_max = S_max;
  x.H_q = H_q;
  x.H_kv = H_kv;
  x.grp = H_q / H_kv;
  x.k = k;
  x.scale_log2 = sm_scale * 1.4426950408889634f;
  x.n_splits = pl.n_splits;
  x.chunks = pl.chunks;
  x.chunks_per_split = pl.chunks_per_split;
  const size_t parts = (size_t)B * T * H_kv * pl.n_splits;
  const size_t o_bytes = ((parts * 16 * d * sizeof(float) + 255) / 256) * 256;
  // Layers share a launch only when one layer's grid is short of two rounds of resident
  // blocks (decode): there the launches are latency-bound and the layers overlap.
  const int per_launch = parts < 1024 ? kAttnMaxLayers : 1;
  for (int l0 = 0; l0 < n_layers; l0 += per_launch) {
    const int nl = n_layers - l0 < per_launch ? n_layers - l0 : per_launch;
    x.layers = nl;
    for (int l = 0; l < kAttnMaxLayers; ++l) {
      const int src = l0 + (l < nl ? l : 0);
      x.q[l] = reinterpret_cast<const uint16_t*>(q[src]);
      x.kc[l] = reinterpret_cast<const uint16_t*>(kc[src]);
      x.vc[l] = reinterpret_cast<const uint16_t*>(vc[src]);
      x.out[l] = reinterpret_cast<uint16_t*>(out[src]);
      x.lse[l] = lse ? lse[src] : nullptr;
      char* part = reinterpret_cast<char*>(ws) + (size_t)(l < nl ? l : 0) * pl.ws_bytes;
      x.part_o[l] = pl.n_splits > 1 ? reinterpret_cast<float*>(part) : nullptr;
      x.part_lse[l] = pl.n_splits > 1 ? reinterpret_cast<float*>(part + o_bytes) : nullptr;
    }
    const size_t per_layer = (size_t)B * T * H_kv * pl.n_splits;
    x.blocks_per_layer = (unsigned)per_layer;
    const dim3 grid((unsigned)(per_layer * nl));
    auto* kern = d == 128 ? (nl > 1 ? &sparse_attn_kernel<128, true> : &sparse_attn_kernel<128, false>)
                          : (nl > 1 ? &sparse_attn_kernel<64, true> : &sparse_attn_kernel<64, false>);
    hipLaunchKernelGGL(kern, grid, dim3(kAttnBlock), 0, stream, x);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (pl.n_splits == 1) continue;
    const int64_t per = (int64_t)B * T * H_q * d;
    const dim3 cgrid((unsigned)((per * nl + 255) / 256));
    if (d == 128)
      hipLaunchKernelGGL(sparse_attn_combine_kernel<128>, cgrid, dim3(256), 0, stream, x, per);
    else
      hipLaunchKernelGGL(sparse_attn_combine_kernel<64>, cgrid, dim3(256), 0, stream, x, per);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* idx,
                              const int32_t* kv_len, int B, int T, int S_max, int H_q, int H_kv,
                              int d, int k, float sm_scale, void* out, float* lse,
                              const AttnPlan& pl, void* ws, hipStream_t stream) {
  return launch_sparse_attn_layers(1, &q, &kc, &vc, idx, kv_len, B, T, S_max, H_q, H_kv, d, k,
                                   sm_scale, &out, &lse, pl, ws, stream);
}

// The backward of n_layers layers over one selection: with atomics, each layer on its own;
// atomic-free, the selection is inverted once per pass of query rows and every layer's
// dV | dK rows are summed per key through that inversion (the layers of an IndexShare group).
hipError_t launch_sparse_attn_bwd_layers(int n_layers, const void* const* q, const void* const* kc,
                                         const void* const* vc, const int32_t* idx,
                                         const int32_t* kv_len, const void* const* out,
                                         const float* const* lse, const void* const* dout, int B,
                                         int T, int S_max, int H_q, int H_kv, int d, int k,
                                         float sm_scale, float* const* dq, float* const* dkc,
                                         float* const* dvc, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  auto args = [&](int l) {
    AttnBwdArgs x{};
    x.q = reinterpret_cast<const uint16_t*>(q[l]);
    x.kc = reinterpret_cast<const uint16_t*>(kc[l]);
    x.vc = reinterpret_cast<const uint16_t*>(vc[l]);
    x.idx = idx;
    x.kv_len = kv_len;
    x.out = reinterpret_cast<const uint16_t*>(out[l]);
    x.lse = lse[l];
    x.dout = reinterpret_cast<const uint16_t*>(dout[l]);
    x.B = B;
    x.T = T;
    x.S_max = S_max;
    x.H_q = H_q;
    x.H_kv = H_kv;
    x.grp = H_q / H_kv;
    x.k = k;
    x.chunks = (k + kChunk - 1) / kChunk;
    x.scale = sm_scale;
    x.scale_log2 = sm_scale * 1.4426950408889634f;
    x.dq = dq[l];
    x.dkc = dkc[l];
    x.dvc = dvc[l];
    return x;
  };
  auto grad = [&](const AttnBwdArgs& x, int64_t rows) {
    const dim3 grid((unsigned)(rows * H_kv));
    if (d == 128)
      hipLaunchKernelGGL(sparse_attn_bwd_kernel<128>, grid, dim3(kAttnBlock), 0, stream, x);
    else
      hipLaunchKernelGGL(sparse_attn_bwd_kernel<64>, grid, dim3(kAttnBlock), 0, stream, x);
  };
  const int64_t all = (int64_t)B * T;
  if (!ws) {
    for (int l = 0; l < n_layers; ++l) {
      AttnBwdArgs x = args(l);
      x.row0 = 0;
      x.contrib = nullptr;
      grad(x, all);
    }
    return hipGetLastError();
  }
  // atomic-free: per pass, the inverted selection, then per layer the pair rows [dV | dK]
  // in bf16 and their key sums
  const size_t row_bytes = (size_t)H_kv * 2 * d * 2;
  const int64_t per_pass = pair_rows_per_pass(B, T, S_max, k, row_bytes, ws_bytes);
  if (per_pass < 1) return hipErrorInvalidValue;
  const PairLayout L = pair_layout(B, S_max, k, per_pass, row_bytes);
  uint16_t* contrib = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + L.contrib);
  for (int64_t r0 = 0; r0 < all; r0 += per_pass) {
    const int64_t rows = std::min(per_pass, all - r0);
    hipError_t e = launch_pair_index(idx, kv_len, T, S_max, k, r0, rows, L, ws, stream);
    if (e != hipSuccess) return e;
    for (int l = 0; l < n_layers; ++l) {
      AttnBwdArgs x = args(l);
      x.row0 = r0;
      x.contrib = contrib;
      grad(x, rows);
      e = launch_pair_reduce(L, ws, 2 * d, H_kv, dvc[l], dkc[l], d, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_sparse_attn_bwd(const void* q, const void* kc, const void* vc, const int32_t* idx,
                                  const int32_t* kv_len, const void* out, const float* lse,
                                  const void* dout, int B, int T, int S_max, int H_q, int H_kv,
                                  int d, int k, float sm_scale, float* dq, float* dkc, float* dvc,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  return launch_sparse_attn_bwd_layers(1, &q, &kc, &vc, idx, kv_len, &out, &lse, &dout, B, T, S_max,
                                       H_q, H_kv, d, k, sm_scale, &dq, &dkc, &dvc, ws, ws_bytes,
                                       stream);
}

hipError_t launch_indexer_kl(const void* q, const void* kc, const int32_t* idx,
                             const int32_t* kv_len, const float* lse, const float* sel_scores,
                             int B, int T, int S_max, int H_q, int H_kv, int d, int k,
                             float sm_scale, float* loss, float* dscores, hipStream_t stream) {
  KlArgs x{};
  x.q = reinterpret_cast<const uint16_t*>(q);
  x.kc = reinterpret_cast<const uint16_t*>(kc);
  x.idx = idx;
  x.kv_len = kv_len;
  x.lse = lse;
  x.sc = sel_scores;
  x.B = B;
  x.T = T;
  x.S_max = S_max;
  x.H_q = H_q;
  x.H_kv = H_kv;
  x.grp = H_q / H_kv;
  x.k = k;
  x.chunks = (k + kChunk - 1) / kChunk;
  x.scale_log2 = sm_scale * 1.4426950408889634f;
  x.loss = loss;
  x.dsc = dscores;
  const size_t blocks = (size_t)B * T;
  if (d == 128)
    hipLaunchKernelGGL(indexer_kl_kernel<128>, dim3((unsigned)blocks), dim3(kAttnBlock), 0, stream, x);
  else
    hipLaunchKernelGGL(indexer_kl_kernel<64>, dim3((unsigned)blocks), dim3(kAttnBlock), 0, stream, x);
  return hipGetLastError();
}

}  // namespace ix
