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

#include "attn_common.h"
#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

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

}  // namespace ix
