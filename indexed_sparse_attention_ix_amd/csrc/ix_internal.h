// Host-side plans and launcher entry points shared by the ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ix.h"

namespace ix {

// How the fused indexer + selection is cut into wave units.
struct TopkPlan {
  int qc;         // queries per wave (4: 4 queries x 4 heads per MFMA column block;
                  //                   1: 1 query  x 16 heads)
  int hc;         // heads per MFMA column block (16 / qc)
  int g;          // MFMA column blocks per key tile (H_I / hc)
  int gmax;       // compiled bound on g
  int qgroups;    // ceil(T / qc) query groups per sequence
  int n_splits;   // key splits per query (1: the wave writes the final selection)
  int split_len;  // keys per split (multiple of 16)
  int cap;        // candidate-buffer entries per (query, split)
  int ksplit;     // entries each split keeps (k when n_splits == 1)
  int fb_cap;     // candidate-buffer entries per (query, split) of the recompute pass (k per split)
  int samp_tiles, fb_samp_tiles;  // key tiles in a starting-threshold sample
  int64_t units;  // wave units = B * qgroups * n_splits
  // workspace: candidates | per-split counts | per-split smallest kept key | query flags
  size_t cand_bytes, cnt_bytes, min_bytes, flag_bytes, ws_bytes;
};

TopkPlan make_topk_plan(const ix_indexer_args& a, int k);

// Sparse attention launch shape.
struct AttnPlan {
  int layers;       // layers per launch: up to 8 share one grid when one layer's grid is small
  int n_splits;     // blocks per (query, kv head); >1 writes partials then combines
  bool light;       // the light kernel (16-row chunks, many waves per CU) for small grids
  int chunks;       // ceil(k / 32), or ceil(k / 16) for the light kernel
  int chunks_per_split;
  size_t part_bytes;  // split partials of one layer of a launch (0 without splits)
  size_t ws_bytes;    // layers * part_bytes
};

// The launch shape for the attention of n_layers layers over one selection (1 for
// sparse_attn_fwd).
AttnPlan make_attn_plan(int B, int T, int H_q, int H_kv, int d, int k, int n_layers);
// The largest workspace the attention of any number of layers needs.
size_t attn_group_ws_bytes(int B, int T, int H_q, int H_kv, int d, int k);

hipError_t launch_ix_score(const ix_indexer_args& a, int t_begin, int t_end, float* scores,
                           hipStream_t stream);
// Debug status words (unsigned long long each, in the order of ix_debug_status).
enum DebugWord {
  kDbgIdxOutOfRange = 0,
  kDbgTopkCompactions,
  kDbgTopkResweeps,
  kDbgTopkSplitRecomputes,
  kDbgTopkOverflow,
  kDbgWords
};

// a.k holds one key row per unit of `pool` positions (1: tokens) and a.S_max counts
// units; a.q_pos0 and a.kv_len count positions.  dbg: the debug status words, or null.
hipError_t launch_ix_topk(const ix_indexer_args& a, int k, const TopkPlan& p, int32_t* idx,
                          float* sel_scores, void* ws, hipStream_t stream, int pool = 1,
                          unsigned long long* dbg = nullptr);
// Debug: adds to dbg[kDbgIdxOutOfRange] the entries of idx [B, T, k] outside [-1, kv_len)
// (kv_len[b] clamped to [0, S_max]; NULL kv_len: S_max).
hipError_t launch_idx_check(const int32_t* idx, const int32_t* kv_len, int B, int T, int S_max,
                            int k, unsigned long long* dbg, hipStream_t stream);
hipError_t launch_pool_keys(const uint8_t* k_I, const int32_t* kv_len, int B, int S_max, int d_I,
                            int pool, uint8_t* k_pooled, hipStream_t stream);
hipError_t launch_expand_blocks(const int32_t* blocks, const int32_t* q_pos0,
                                const int32_t* kv_len, int B, int T, int S_max, int k_blocks,
                                int pool, int32_t* idx, hipStream_t stream);
hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* idx,
                              const int32_t* kv_len, int B, int T, int S_max, int H_q, int H_kv,
                              int d, int k, float sm_scale, void* out, float* lse,
                              const AttnPlan& p, void* ws, hipStream_t stream);

// The attention of n_layers layers over one selection, pl = make_attn_plan(..., n_layers):
// pl.layers layers per launch; layer l of a launch uses ws + l * pl.part_bytes for its
// split partials.
hipError_t launch_sparse_attn_layers(int n_layers, const void* const* q, const void* const* kc,
                                     const void* const* vc, const int32_t* idx,
                                     const int32_t* kv_len, int B, int T, int S_max, int H_q,
                                     int H_kv, int d, int k, float sm_scale, void* const* out,
                                     float* const* lse, const AttnPlan& pl, void* ws,
                                     hipStream_t stream);
// Atomic-free key gradients (pair_reduce.hip): workspace layout for passes of `rows` query
// rows whose pairs carry row_bytes of gradient rows (bf16 or fp32) each.
struct PairLayout {
  int64_t n_keys, nparts;
  int64_t n_blk, rows_per_blk, n_slots;  // row blocks of the pass; (key, block) counters
  size_t off, cnt, cur, part_sum, part, inv, contrib, total;
};
PairLayout pair_layout(int B, int S_max, int k, int64_t rows, size_t row_bytes);
int64_t pair_rows_per_pass(int B, int T, int S_max, int k, size_t row_bytes, size_t ws_bytes);
// Offsets and the inverted selection of query rows [row0, row0 + rows).
hipError_t launch_pair_index(const int32_t* idx, const int32_t* kv_len, int T, int S_max, int k,
                             int64_t row0, int64_t rows, const PairLayout& L, void* ws,
                             hipStream_t stream);
// Per-key sums of the pass's pair rows (row_width elements per (pair, head), bf16, or fp32
// with f32_rows; H heads), first half added to dst_a, second half to dst_b, at row
// (key * H + head) of `stride` floats.
hipError_t launch_pair_reduce(const PairLayout& L, const void* ws, int row_width, bool f32_rows,
                              int H, float* dst_a, float* dst_b, int64_t stride,
                              hipStream_t stream);
hipError_t launch_sparse_attn_bwd_layers(int n_layers, const void* const* q, const void* const* kc,
                                         const void* const* vc, const int32_t* idx,
                                         const int32_t* kv_len, const void* const* out,
                                         const float* const* lse, const void* const* dout, int B,
                                         int T, int S_max, int H_q, int H_kv, int d, int k,
                                         float sm_scale, float* const* dq, float* const* dkc,
                                         float* const* dvc, bool f32_rows, void* ws,
                                         size_t ws_bytes, hipStream_t stream);
hipError_t launch_sparse_attn_bwd(const void* q, const void* kc, const void* vc, const int32_t* idx,
                                  const int32_t* kv_len, const void* out, const float* lse,
                                  const void* dout, int B, int T, int S_max, int H_q, int H_kv,
                                  int d, int k, float sm_scale, float* dq, float* dkc, float* dvc,
                                  bool f32_rows, void* ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_indexer_kl(const void* q, const void* kc, const int32_t* idx,
                             const int32_t* kv_len, const float* lse, const float* sel_scores,
                             int B, int T, int S_max, int H_q, int H_kv, int d, int k,
                             float sm_scale, float* loss, float* dscores, hipStream_t stream);
hipError_t launch_indexer_bwd(const uint8_t* qI, const uint8_t* kI, const float* w,
                              const int32_t* kv_len, const int32_t* idx, const float* dscores,
                              int B, int T, int S_max, int H_I, int d_I, int k, float* dq,
                              float* dw, float* dk, bool f32_rows, void* ws, size_t ws_bytes,
                              hipStream_t stream);
hipError_t launch_append_kv(const float* k_I_new, const void* K_new, const void* V_new,
                            const int32_t* pos0, int B, int T_new, int S_max, int d_I, int H_kv,
                            int d, uint8_t* k_I_cache, void* K_cache, void* V_cache,
                            hipStream_t stream);

}  // namespace ix
