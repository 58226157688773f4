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
// The four waves' (m, l, O) are merged through LDS at the end.  Small batches (decode) take
// a lighter variant of the kernel, may split the selection over several blocks and merge the
// normalised partials by lse; when one layer's grid is that small, the layers of an
// IndexShare group share one launch (each block serves one layer; the split count follows the
// launch's total grid, so a layer's result equals the single-layer call's up to the rounding
// of the partials' merge, and bit for bit when both use the same split count).
#include <algorithm>

#include "attn_common.h"
#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

// Layers whose attention one launch can run: each block serves one layer.
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

// End of a block: the four waves' (m, l, O^T) merged through LDS (wave w's O^T staged at
// lds + w * wave_bytes as [head][d] floats; ml: each wave's per-head m and l), then the
// normalised output and lse, or with splits this block's normalised partial and its lse.
template <int D, bool ML>
__device__ __forceinline__ void finish_block(const AttnArgs& p, int layer, int64_t rk, int kvh,
                                             int64_t row, int split, const f32x4 (&o)[D / 16],
                                             float m_run, float l_run, unsigned char* lds,
                                             size_t wave_bytes, float (*ml)[2][16]) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  // per-head l: sum the four lane groups' shares
  l_run = sum_across_rows(l_run);
  __syncthreads();
  float* os = reinterpret_cast<float*>(lds + wid * wave_bytes);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) os[r16 * D + 16 * nt + 4 * lg + i] = o[nt][i];
  if (lg == 0) {
    ml[wid][0][r16] = m_run;
    ml[wid][1][r16] = l_run;
  }
  __syncthreads();

  const float ln2 = 0.69314718055994530942f;
  for (int e = threadIdx.x; e < 16 * D; e += kAttnBlock) {
    const int h = e / D, dcol = e % D;
    if (h >= p.grp) continue;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, ml[w][0][h]);
    float L = 0.f, acc = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = ml[w][0][h];
        const float f = mw == -__builtin_inff() ? 0.f : exp2f(mw - M);
        L += f * ml[w][1][h];
        acc += f * reinterpret_cast<const float*>(lds + w * wave_bytes)[h * D + dcol];
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
  __shared__ bf16x8 q_lds[MC][kWave];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  // XCD-aware order: the hardware deals consecutive blocks to the 8 XCDs in turn, so
  // block i runs on XCD i % 8; give each XCD a contiguous range of rows so nearby
  // queries (which tend to select overlapping keys) share one L2.
  unsigned bid = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
  const int layer = ML ? __builtin_amdgcn_readfirstlane((int)(bid / p.blocks_per_layer)) : 0;
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
  // uniform: the buffer bounds built on it stay in scalar registers
  kvl = __builtin_amdgcn_readfirstlane(kvl < 0 ? 0 : (kvl > p.S_max ? p.S_max : kvl));

  // Q as the B operand of S^T = K Q^T: column = head, depth slice [32m + 8lg, +8).  The four
  // waves use the same operands: wave 0 stages them in LDS, in lane order, and every chunk
  // reads them from there (registers hold the rows in flight instead).
  const bool hvalid = r16 < p.grp;
  if (wid == 0) {
    const int head = kvh * p.grp + (hvalid ? r16 : 0);
    const uint16_t* qrow = q_l + ((size_t)row * p.H_q + head) * D;
#pragma unroll
    for (int m = 0; m < MC; ++m)
      q_lds[m][lane] = hvalid ? load_bf16x8(qrow + 32 * m + 8 * lg) : (bf16x8){};
  }
  __syncthreads();

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

  // Entry e_lane of chunk c as stored (lanes 32..63 repeat lanes 0..31), 0 past the row or the
  // split (such loads fall outside the buffer and fetch nothing).
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(irow, (uint32_t)p.k * 4u);
  const int e_lane = lane & (kChunk - 1);
  auto raw_of = [&](int c) -> int {
    const uint32_t off = c < c_end ? (uint32_t)(c * kChunk + e_lane) * 4u : 0x80000000u;
    return __builtin_amdgcn_raw_buffer_load_b32(irs, (int)off, 0, 0);
  };
  // Gathers the rows of chunk c, whose raw entries are j, into (kd, vd): lane (rho, s) takes
  // the keys of slots rho * NI + i from the lanes that hold them.  Returns the chunk's slot
  // mask (bit n: slot n holds a valid key; padding, past the row and not visible are not).
  i32x4 kdA[NI], vdA[NI], kdB[NI], vdB[NI];
  auto issue = [&](int c, int j, i32x4 (&kd)[NI], i32x4 (&vd)[NI]) -> uint32_t {
    const int e = c * kChunk + e_lane;
    const bool valid = c < c_end && e < p.k && j >= 0 && j < kvl;
    // the row's byte offset, formed once by the lane that holds the entry (an invalid entry
    // reads past the buffer: 0x80000000 plus a piece offset stays out of range)
    const uint32_t roff = valid ? (uint32_t)j * kv_stride_b : 0x80000000u;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t off = (uint32_t)__shfl((int)roff, rho * NI + i) + 16u * s;
      kd[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
      vd[i] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, 0));
    }
    return (uint32_t)ballot64(valid);
  };

  // Two register sets of chunk rows alternate, each serving every other chunk of the wave:
  // while a chunk is computed, the gathers of the next two are in flight.  A set's raw entries
  // for its next chunk are loaded right after its rows, so the wait for them, a step later,
  // leaves the other set's rows in flight; past the split the loads are issued all the same
  // (they fetch nothing), which keeps the wait counts exact.
  constexpr int W = kAttnWaves;
  const int c0 = c_begin + wid;
  int jA = raw_of(c0), jB = raw_of(c0 + W);
  uint32_t maskA = issue(c0, jA, kdA, vdA);
  jA = raw_of(c0 + 2 * W);
  uint32_t maskB = issue(c0 + W, jB, kdB, vdB);
  jB = raw_of(c0 + 3 * W);

  // chunk c, whose rows are in (kd, vd): stage them (bank-swizzled), refill the set with
  // chunk c + 2W, then compute
  auto step = [&](int c, i32x4 (&kd)[NI], i32x4 (&vd)[NI], uint32_t& mask, int& jr)
      __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      *reinterpret_cast<i32x4*>(kst + woff[j]) = kd[j];
      *reinterpret_cast<i32x4*>(vst + woff[j]) = vd[j];
    }
    const uint32_t vmask = mask;
    mask = issue(c + 2 * W, jr, kd, vd);
    jr = raw_of(c + 4 * W);
    lds_wait();

    // S^T tiles: lane holds keys 16*tt + 4*lg + i for head r16
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(kst + koff[m]);
      const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(kst + koff[m] + 16 * ROWB);
      const bf16x8 qb = q_lds[m][lane];
      s0 = mfma_bf16_16x16x32(ka0, qb, s0);
      s1 = mfma_bf16_16x16x32(ka1, qb, s1);
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
    const float alpha = (any && m_run != -__builtin_inff()) ? exp2_hw(m_run - m_new) : (any ? 0.f : 1.f);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = (x[e] != -__builtin_inff()) ? exp2_hw(x[e] - m_new) : 0.f;
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
      for (int e = 0; e < 4; ++e) pk[e] = (int)pack_bf16x2(pr[2 * e], pr[2 * e + 1]);
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
  // pairs of steps, then a last one if the wave has an odd number of chunks: every path back
  // to the loop head has issued the same loads
  int c = c0;
  for (; c + W < c_end; c += 2 * W) {
    step(c, kdA, vdA, maskA, jA);
    step(c + W, kdB, vdB, maskB, jB);
  }
  if (c < c_end) step(c, kdA, vdA, maskA, jA);

  finish_block<D, ML>(p, layer, rk, kvh, row, split, o, m_run, l_run, &stage_all[0][0][0],
                      sizeof(stage_all[0]), ml_all);
}

// Launches of few query rows (decode) gather their rows from HBM.  This variant keeps the math
// of the kernel above but takes 16-row chunks and loads each K row straight into the MFMA
// operand registers (lane (g, r) reads row r's 16-byte pieces 4m + g, the A-operand layout of
// S^T = K Q^T; no LDS); only V is staged (4 KiB per wave at d = 128) for the transposing read
// of O^T += V^T P^T (bf16 16x16x16).  Each wave keeps the rows of its next two chunks in
// registers, so their gathers overlap a chunk's arithmetic: 158-167 VGPRs and 32 KiB of LDS per
// block.  On the decode step it beats the kernel above (14.1 against 17 us per layer for a
// 4-layer launch; loading K whole, as V, and staging it in LDS as well takes 16.4 us).
constexpr int kLightChunk = 16;

template <int D, bool ML>
__global__ __launch_bounds__(kAttnBlock, 3) void sparse_attn_light_kernel(AttnArgs p) {
  constexpr int MC = D / 32;               // depth tiles of the QK^T product
  constexpr int NT = D / 16;               // 16-row tiles of O^T
  constexpr int ROWB = D * 2;              // bytes per K or V row
  constexpr int PI = ROWB / 16;            // 16-byte pieces per row
  constexpr int RPI = kWave / PI;          // rows per 64-lane load
  constexpr int NIV = kLightChunk / RPI;   // V loads per chunk per lane
  constexpr int WAVE_LDS = 16 * D * 4;     // per wave: the V stage, then O^T for the merge
  static_assert(kLightChunk * ROWB <= WAVE_LDS, "V stage");
  __shared__ __attribute__((aligned(16))) unsigned char lds_all[kAttnWaves][WAVE_LDS];
  __shared__ float ml_all[kAttnWaves][2][16];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  unsigned bid = blockIdx.x;
  if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
  const int layer = ML ? __builtin_amdgcn_readfirstlane((int)(bid / p.blocks_per_layer)) : 0;
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
  // uniform: the buffer bounds built on it stay in scalar registers
  kvl = __builtin_amdgcn_readfirstlane(kvl < 0 ? 0 : (kvl > p.S_max ? p.S_max : kvl));

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
  unsigned char* vst = lds_all[wid];

  // V stage: lane (rho, s) of load j fetches piece s of slot n = rho * NIV + j
  const int rho = lane / PI, s = lane % PI;
  uint32_t woff[NIV];
#pragma unroll
  for (int j = 0; j < NIV; ++j) {
    const int n = rho * NIV + j;
    woff[j] = (uint32_t)(n * ROWB + 16 * (s ^ stage_swz<D>(n)));
  }
  // transposed V read: slot 4lg + r16/4, logical bytes [32nt + 8(r16 & 3), +8)
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
  // Entry r16 of chunk c (the same in the four lane groups) as stored, 0 past the row or the
  // split (such loads fall outside the buffer and fetch nothing).
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(irow, (uint32_t)p.k * 4u);
  auto raw_of = [&](int c) -> int {
    const uint32_t off = c < c_end ? (uint32_t)(c * kLightChunk + r16) * 4u : 0x80000000u;
    return __builtin_amdgcn_raw_buffer_load_b32(irs, (int)off, 0, 0);
  };
  // the key of a raw entry of chunk c, -1 if padding, past the row or not visible
  auto key_of = [&](int c, int j) -> int {
    const int e = c * kLightChunk + r16;
    return (c < c_end && e < p.k && j >= 0 && j < kvl) ? j : -1;
  };
  // one chunk in registers: its K rows as A operands (lane: row r16, pieces 4m + lg), its V
  // rows for the stage, and which of its 16 keys are valid.  The rows are loaded
  // non-temporal: this kernel serves decode-size grids, whose caches (gigabytes per layer)
  // come from HBM and are read once per step
  struct Rows {
    bf16x8 ka[MC];
    i32x4 vd[NIV];
    uint32_t mask;
  };
  auto issue = [&](int jk, Rows& r) {
    // the row's byte offset, formed once by the lane that holds the entry (an invalid entry
    // reads past the buffer: 0x80000000 plus a piece offset stays out of range)
    const uint32_t roff = jk >= 0 ? (uint32_t)jk * kv_stride_b : 0x80000000u;
    const uint32_t kbase = roff + 16u * lg;
#pragma unroll
    for (int m = 0; m < MC; ++m)
      r.ka[m] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(kbase + 64u * m), 0, kLoadNT));
#pragma unroll
    for (int j = 0; j < NIV; ++j) {
      const uint32_t off = (uint32_t)__shfl((int)roff, rho * NIV + j) + 16u * s;
      r.vd[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, (int)off, 0, kLoadNT));
    }
    r.mask = (uint32_t)ballot64(jk >= 0) & 0xFFFFu;  // lanes 0..15 hold keys 0..15
  };

  // Each register set (rows and the raw entries of its next chunk) serves every other chunk
  // of the wave.  A set's entries are loaded right after its rows, so the wait for them, one
  // step later, leaves the other set's rows in flight; past the split the loads are issued
  // all the same (they fetch nothing), which keeps the wait counts exact.
  constexpr int W = kAttnWaves;
  const int c0 = c_begin + wid;
  Rows rA, rB;
  int jA = raw_of(c0), jB = raw_of(c0 + W);
  issue(key_of(c0, jA), rA);
  jA = raw_of(c0 + 2 * W);
  issue(key_of(c0 + W, jB), rB);
  jB = raw_of(c0 + 3 * W);

  // chunk c, whose rows are in r: S^T from the K operands, V staged, then r refilled with
  // chunk c + 2W (its gathers in flight during this chunk's softmax and O^T update, with
  // those of chunk c + W)
  auto step = [&](int c, Rows& r, int& jr) __attribute__((always_inline)) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < MC; ++m) s0 = mfma_bf16_16x16x32(r.ka[m], qb[m], s0);
#pragma unroll
    for (int j = 0; j < NIV; ++j) *reinterpret_cast<i32x4*>(vst + woff[j]) = r.vd[j];
    const uint32_t vmask = r.mask;
    issue(key_of(c + 2 * W, jr), r);
    jr = raw_of(c + 4 * W);
    lds_wait();

    float x[4];
    float mloc = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (vmask >> (4 * lg + i)) & 1u;
      x[i] = ok ? s0[i] * p.scale_log2 : -__builtin_inff();
      mloc = fmaxf(mloc, x[i]);
    }
    mloc = max_across_rows(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const bool any = m_new != -__builtin_inff();
    const float alpha = (any && m_run != -__builtin_inff()) ? exp2_hw(m_run - m_new) : (any ? 0.f : 1.f);
    float pr[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = (x[i] != -__builtin_inff()) ? exp2_hw(x[i] - m_new) : 0.f;
      psum += pr[i];
    }
    const i16x4 pb = __builtin_bit_cast(
        i16x4, (uint32_t __attribute__((ext_vector_type(2)))){pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // O^T += V^T P^T: P^T (keys 4lg..4lg+3 of head r16) is the B operand as the lane holds it
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[nt][i] *= alpha;
      o[nt] = mfma_bf16_16x16x16(lds_read_tr16(vst + voff[nt]), pb, o[nt]);
    }
    lds_wait();  // the stage is rewritten by the next chunk
  };
  // pairs of steps, then a last one if the wave has an odd number of chunks: every path back
  // to the loop head has issued the same loads
  int c = c0;
  for (; c + W < c_end; c += 2 * W) {
    step(c, rA, jA);
    step(c + W, rB, jB);
  }
  if (c < c_end) step(c, rA, jA);

  finish_block<D, ML>(p, layer, rk, kvh, row, split, o, m_run, l_run, &lds_all[0][0],
                      sizeof(lds_all[0]), ml_all);
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

}  // namespace

// Grids of fewer than 1024 blocks per layer (decode) gather from HBM: one launch then serves
// up to 8 layers with the light kernel, each selection split over as many blocks as make the
// launch about one block per CU (256), each wave getting at least two chunks.  Measured on the
// 64-sequence decode step with the caches cold: the 4 layers in one launch take 14.1 us per
// layer at 1 block per query (2, 3, 4 and 6 blocks: 15.8-15.9, 16.5, 16.7 and 18.2 us; more
// blocks put more requests in flight and add the combine launch), one layer 26.8 us at 4
// blocks per query (2, 3, 6 and 8: 28.7, 27.2, 30.5 and 29.9 us; the kernel above: 31.2 us).
// Larger grids (prefill) take the kernel above, faster there (128K: 13.7 against 15.5 ms).
AttnPlan make_attn_plan(int B, int T, int H_q, int H_kv, int d, int k, int n_layers) {
  (void)H_q;
  AttnPlan p{};
  p.chunks = (k + kChunk - 1) / kChunk;
  const int64_t base = (int64_t)B * T * H_kv;
  int ns = 1;
  p.layers = 1;
  p.light = false;
  if (base > 0 && base < 1024) {
    p.layers = n_layers < kAttnMaxLayers ? (n_layers < 1 ? 1 : n_layers) : kAttnMaxLayers;
    p.light = true;
    p.chunks = (k + kLightChunk - 1) / kLightChunk;
    const int64_t grid = base * p.layers;
    const int64_t target = 256;
    int64_t want = (target + grid / 2) / grid;
    int64_t by_chunks = p.chunks / (2 * kAttnWaves);
    if (by_chunks < 1) by_chunks = 1;
    if (want < 1) want = 1;
    ns = (int)(want < by_chunks ? want : by_chunks);
  }
  p.n_splits = ns;
  p.chunks_per_split = (p.chunks + ns - 1) / ns;
  if (ns > 1) {
    const size_t parts = (size_t)base * ns;
    const size_t o_bytes = parts * 16 * d * sizeof(float);
    const size_t l_bytes = parts * 16 * sizeof(float);
    p.part_bytes = ((o_bytes + 255) / 256) * 256 + ((l_bytes + 255) / 256) * 256;
  }
  p.ws_bytes = (size_t)p.layers * p.part_bytes;
  return p;
}

size_t attn_group_ws_bytes(int B, int T, int H_q, int H_kv, int d, int k) {
  size_t m = 0;
  for (int n = 1; n <= kAttnMaxLayers; ++n) {
    const size_t w = make_attn_plan(B, T, H_q, H_kv, d, k, n).ws_bytes;
    m = w > m ? w : m;
  }
  return m;
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
  const int per_launch = pl.layers;
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
      char* part = reinterpret_cast<char*>(ws) + (size_t)(l < nl ? l : 0) * pl.part_bytes;
      x.part_o[l] = pl.n_splits > 1 ? reinterpret_cast<float*>(part) : nullptr;
      x.part_lse[l] = pl.n_splits > 1 ? reinterpret_cast<float*>(part + o_bytes) : nullptr;
    }
    const size_t per_layer = (size_t)B * T * H_kv * pl.n_splits;
    x.blocks_per_layer = (unsigned)per_layer;
    const dim3 grid((unsigned)(per_layer * nl));
    auto* kern =
        pl.light
            ? (d == 128 ? (nl > 1 ? &sparse_attn_light_kernel<128, true> : &sparse_attn_light_kernel<128, false>)
                        : (nl > 1 ? &sparse_attn_light_kernel<64, true> : &sparse_attn_light_kernel<64, false>))
            : (d == 128 ? &sparse_attn_kernel<128, false> : &sparse_attn_kernel<64, false>);
    // (a launch of the light kernel may hold a single layer; the kernel above runs one layer
    // per launch: only small grids share launches, and those take the light kernel)
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

}  // namespace ix
