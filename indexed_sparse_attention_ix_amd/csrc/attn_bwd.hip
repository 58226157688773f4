// The training side of the sparse attention: its gradients over the selection and the
// indexer's KL objective against the attention distribution (the twiscan post on GLM-5.2's
// IndexShare: the indexer learns to imitate the attention distribution through a KL loss).
// Kernel shapes and the staging of K/V rows follow the forward kernel in sparse_attn.hip.
#include <algorithm>

#include "attn_common.h"
#include "ix_common.h"
#include "ix_internal.h"

namespace ix {

namespace {

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
  void* contrib;      // non-null: per-pair dV | dK rows instead of atomics
};

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
// F32ROWS: the pair rows (p.contrib, required) in fp32; otherwise in bf16, or atomics
// without p.contrib.
template <int D, bool F32ROWS = false>
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
      pr[i] = ok0 ? exp2_hw(s0[i] * p.scale_log2 - lse2) : 0.f;
      pr[4 + i] = ok1 ? exp2_hw(s1[i] * p.scale_log2 - lse2) : 0.f;
      ds[i] = pr[i] * (dp0[i] - Dh);
      ds[4 + i] = pr[4 + i] * (dp1[i] - Dh);
    }

    // dq^T += K^T dS^T: dS^T as the B operand (column = head r16)
    {
      i32x4 dk;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dk[e] = (int)pack_bf16x2(ds[2 * e], ds[2 * e + 1]);
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
    // (with a pair buffer) each selected pair's dV | dK rows in bf16 or fp32, staged in the
    // K / V stage (no longer read in this chunk) and written in pair order, non-temporal: the
    // rows (tens of GB) are read back once by the key sums, and cached they would evict the
    // K / V rows this kernel gathers
    if constexpr (F32ROWS) {
      // fp32: the dV rows, then the dK rows, each a [pair][D] tile filling the stage.  The
      // 16-byte pieces of a row are swizzled by the pair's lane group (pair bits 2..3), so
      // the four lane groups' writes of one instruction fall in different banks.
      float* cf = reinterpret_cast<float*>(stage_all[wid][0]);
      static_assert(kChunk * D * 4 <= 2 * kChunk * ROWB, "fp32 pair staging");
      constexpr int kPieces = D / 4;  // 16-byte pieces of one pair's dV (or dK) row
      float* dst0 = reinterpret_cast<float*>(p.contrib) +
                    ((size_t)(row - p.row0) * p.k * p.H_kv + kvh) * 2 * D;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)((half ? pts : ptp) + pt_r + 16 * tt));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 v = mfma_bf16_16x16x16(a, half ? qB[nt] : doB[nt], z);
            const int piece = (4 * nt + (r16 >> 2)) ^ (4 * lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) cf[(16 * tt + 4 * lg + i) * D + 4 * piece + (r16 & 3)] = v[i];
          }
        }
        lds_wait();
        for (int q2 = lane; q2 < kChunk * kPieces; q2 += kWave) {
          const int e = q2 / kPieces, pc = q2 % kPieces;
          const int ent = c * kChunk + e;
          if (ent < p.k) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(cf + e * D + 4 * (pc ^ (4 * ((e >> 2) & 3))));
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst0 + (size_t)ent * p.H_kv * 2 * D + half * D + 4 * pc));
          }
        }
        lds_wait();
      }
      continue;
    }
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
      uint16_t* dst0 = reinterpret_cast<uint16_t*>(p.contrib) +
                       ((size_t)(row - p.row0) * p.k * p.H_kv + kvh) * 2 * D;
      for (int q2 = lane; q2 < kChunk * kPieces; q2 += kWave) {
        const int e = q2 / kPieces, pc = q2 % kPieces;
        const int ent = c * kChunk + e;
        if (ent < p.k) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(cb + (size_t)e * 2 * D + 8 * pc);
          __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(dst0 + (size_t)ent * p.H_kv * 2 * D + 8 * pc));
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

  // Entry e_lane of chunk c as stored (lanes 32..63 repeat lanes 0..31), 0 past the row; it
  // is loaded a chunk ahead and checked where the rows are issued, so the wait for it does
  // not take the rows issued just before it.
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(irow, (uint32_t)p.k * 4u);
  const int e_lane = lane & (kChunk - 1);
  auto raw_of = [&](int c) -> int {
    const uint32_t off = c < p.chunks ? (uint32_t)(c * kChunk + e_lane) * 4u : 0x80000000u;
    return __builtin_amdgcn_raw_buffer_load_b32(irs, (int)off, 0, 0);
  };
  auto key_of = [&](int c, int j) -> int {
    const int e = c * kChunk + e_lane;
    return (c < p.chunks && e < p.k && j >= 0 && j < kvl) ? j : -1;
  };
  // the K rows (KV head kvh) of the chunk whose keys, one per lane e_lane, are `key`: lane
  // (rho, s) takes slots rho * NI + j from the lanes that hold them
  i32x4 kd[NI];
  auto issue_rows = [&](int key, int kvh) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int jv = __shfl(key, rho * NI + j);
      const uint32_t off = jv >= 0 ? (uint32_t)jv * kv_stride_b + (uint32_t)(kvh * ROWB) + 16u * s
                                   : 0x80000000u;
      kd[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)off, 0, 0));
    }
  };

  load_head_data(0);
  const int c0 = wid;
  int key_c = key_of(c0, raw_of(c0));
  uint32_t mask_c = (uint32_t)ballot64(key_c >= 0);  // bit n: slot n holds a valid key
  issue_rows(key_c, 0);
  int jn = raw_of(c0 + kAttnWaves);

  for (int c = c0; c < p.chunks; c += kAttnWaves) {
    const uint32_t vmask = mask_c;
    float u0 = 0.f, u1 = 0.f;  // this lane's heads, keys r16 and 16 + r16
    for (int kvh = 0; kvh < p.H_kv; ++kvh) {
#pragma unroll
      for (int j = 0; j < NI; ++j) *reinterpret_cast<i32x4*>(kst + woff[j]) = kd[j];
      if (kvh + 1 < p.H_kv) {
        issue_rows(key_c, kvh + 1);
      } else {  // past the last chunk the keys are -1 and nothing is fetched
        key_c = key_of(c + kAttnWaves, jn);
        mask_c = (uint32_t)ballot64(key_c >= 0);
        issue_rows(key_c, 0);
        jn = raw_of(c + 2 * kAttnWaves);
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
        u0 += exp2_hw(s0[i] * p.scale_log2 - lse2[i]);
        u1 += exp2_hw(s1[i] * p.scale_log2 - lse2[i]);
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

// The backward of n_layers layers over one selection: with atomics, each layer on its own;
// atomic-free, the selection is inverted once per pass of query rows and every layer's
// dV | dK rows are summed per key through that inversion (the layers of an IndexShare group).
hipError_t launch_sparse_attn_bwd_layers(int n_layers, const void* const* q, const void* const* kc,
                                         const void* const* vc, const int32_t* idx,
                                         const int32_t* kv_len, const void* const* out,
                                         const float* const* lse, const void* const* dout, int B,
                                         int T, int S_max, int H_q, int H_kv, int d, int k,
                                         float sm_scale, float* const* dq, float* const* dkc,
                                         float* const* dvc, bool f32_rows, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
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
  auto grad = [&](const AttnBwdArgs& x, int64_t rows, bool f32) {
    const dim3 grid((unsigned)(rows * H_kv));
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kAttnBlock), 0, stream, x); };
    if (d == 128)
      f32 ? go(sparse_attn_bwd_kernel<128, true>) : go(sparse_attn_bwd_kernel<128>);
    else
      f32 ? go(sparse_attn_bwd_kernel<64, true>) : go(sparse_attn_bwd_kernel<64>);
  };
  const int64_t all = (int64_t)B * T;
  if (!ws) {
    for (int l = 0; l < n_layers; ++l) {
      AttnBwdArgs x = args(l);
      x.row0 = 0;
      x.contrib = nullptr;
      grad(x, all, false);
    }
    return hipGetLastError();
  }
  // atomic-free: per pass, the inverted selection, then per layer the pair rows [dV | dK]
  // (bf16 or fp32) and their key sums
  const size_t row_bytes = (size_t)H_kv * 2 * d * (f32_rows ? 4 : 2);
  const int64_t per_pass = pair_rows_per_pass(B, T, S_max, k, row_bytes, ws_bytes);
  if (per_pass < 1) return hipErrorInvalidValue;
  const PairLayout L = pair_layout(B, S_max, k, per_pass, row_bytes);
  void* contrib = reinterpret_cast<char*>(ws) + L.contrib;
  for (int64_t r0 = 0; r0 < all; r0 += per_pass) {
    const int64_t rows = std::min(per_pass, all - r0);
    hipError_t e = launch_pair_index(idx, kv_len, T, S_max, k, r0, rows, L, ws, stream);
    if (e != hipSuccess) return e;
    for (int l = 0; l < n_layers; ++l) {
      AttnBwdArgs x = args(l);
      x.row0 = r0;
      x.contrib = contrib;
      grad(x, rows, f32_rows);
      e = launch_pair_reduce(L, ws, 2 * d, f32_rows, H_kv, dvc[l], dkc[l], d, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_sparse_attn_bwd(const void* q, const void* kc, const void* vc, const int32_t* idx,
                                  const int32_t* kv_len, const void* out, const float* lse,
                                  const void* dout, int B, int T, int S_max, int H_q, int H_kv,
                                  int d, int k, float sm_scale, float* dq, float* dkc, float* dvc,
                                  bool f32_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  return launch_sparse_attn_bwd_layers(1, &q, &kc, &vc, idx, kv_len, &out, &lse, &dout, B, T, S_max,
                                       H_q, H_kv, d, k, sm_scale, &dq, &dkc, &dvc, f32_rows, ws,
                                       ws_bytes, stream);
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
