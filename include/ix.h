/*
 * ix.h -- C ABI of the indexed sparse-attention library (libix.so, gfx950).
 *
 * The path: an FP8 indexer scores every causal key for each query, the k best keys
 * are kept, and attention runs over only the kept K/V rows; under IndexShare one
 * selection serves a group of sparse layers.
 *   Stage 1 (coarse scoring) and Stage 2 (fine selection, k = 2048 at 1M context):
 *     "GLM 5.2: How Four Co-Designed Mechanisms Beat Raw Scale", Part II,
 *     section "DeepSeek Sparse Attention".
 *   The indexer runs in FP8, scores the keys and keeps the top-k, and one
 *   indexer's selection is shared across a group of 4 layers: the twiscan post on
 *   GLM-5.2's IndexShare.
 *   Selection computed once per block of 4 layers and shared across the block:
 *     same irys.ai page, section "IndexShare: Amortizing the Indexer".
 * Concrete indexer form implemented here: for query token t and key token s,
 *     score(t,s) = sum_h w[t,h] * max(0, sum_c q_I[t,h,c] * k_I[s,c])
 * with FP8 (OCP e4m3) q_I/k_I, fp32 w, fp32 accumulation.
 * Accuracy of a score: within about eps * sum_h |w_h| sum_c |q_I[t,h,c] k_I[s,c]|, eps the
 * FP8 matrix core's relative error (measured below 2.4e-4).  With 64 indexer heads and
 * more than 3 query rows, a group of 4 query rows whose head weights are all >= 0 takes
 * the head sum as 1/2 sum_h w_h |x_h| + 1/2 k . u, u = sum_h w_h q_I[t,h,:] in four scaled
 * e4m3 terms (about 1.05x that bound).  Either way a key whose every head dot product is
 * <= 0 scores exactly 0 wherever the top-k could still keep it, and in ix_score always.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE memory owned by the caller; the library never
 *     allocates, frees or synchronises.  Every call is asynchronous on `stream`
 *     (NULL = the default stream).  Tensors are dense row-major with the listed
 *     shapes (innermost dimension last); FP8 rows must be 16-byte aligned, bf16 rows
 *     16-byte aligned (true for any contiguous tensor from a hipMalloc'd base).
 *   - Visibility: query t of sequence b sits at position q_pos0[b] + t and sees the
 *     keys s with s <= q_pos0[b] + t and s < kv_len[b] (its own key included):
 *     n_t = clamp(q_pos0[b] + t + 1, 0, min(kv_len[b], S_max)).
 *   - Arguments are validated before anything is launched.  On a non-OK status the
 *     outputs are untouched (IX_ERR_HIP: launch failure, outputs undefined), and
 *     ix_last_error() returns a message for the calling thread.  No exception or
 *     abort crosses the ABI.
 *   - B == 0 or T == 0 is a valid empty call: IX_OK, nothing launched.
 *   - Supported shapes: d_I in {64,128}; H_I a multiple of 4 in [4,64];
 *     d in {64,128}; H_q a multiple of H_kv with H_q/H_kv <= 16; 1 <= k <= 2048;
 *     one sequence's indexer keys (S_max*d_I bytes) below 2 GiB and its K and V
 *     caches (S_max*H_kv*d*2 bytes each) within 2 GiB.
 *     One call runs each kernel as one launch, and a launch counts its work-items in
 *     32 bits.  Hence at most 2^24 - 1 query rows per indexer call (B*T), per attention
 *     call (B*T*H_kv) and per append (B*T_new).  Likewise at most 2^32 - 256 expanded
 *     entries (B*T*k_blocks*pool) for ix_topk_pooled, and at most 2^32 - 256 key pieces
 *     (B*ceil(S_max/pool)*d_I/8) for ix_pool_keys.
 *     Other shapes return IX_ERR_UNSUPPORTED (no fallback path exists).
 *   - Calls are re-entrant; concurrent calls must not share a workspace.
 */
#ifndef IX_H
#define IX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

typedef enum ix_status {
  IX_OK = 0,
  IX_ERR_INVALID = -1,     /* null pointer, negative size, bad range, bad alignment */
  IX_ERR_UNSUPPORTED = -2, /* shape outside the supported set */
  IX_ERR_WORKSPACE = -3,   /* workspace missing or smaller than *_workspace_bytes() */
  IX_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} ix_status;

/* Indexer inputs (Stage 1 of "DeepSeek Sparse Attention").  All device pointers. */
typedef struct ix_indexer_args {
  const uint8_t *q;      /* [B, T, H_I, d_I]  FP8 e4m3 indexer queries             */
  const uint8_t *k;      /* [B, S_max, d_I]   FP8 e4m3 indexer keys, one row per key
                                              token, shared by all H_I heads        */
  const float *w;        /* [B, T, H_I]       fp32 head weights                      */
  const int32_t *q_pos0; /* [B] position of query t = 0 (query t at q_pos0[b] + t)   */
  const int32_t *kv_len; /* [B] valid keys per sequence (clamped to S_max)           */
  int32_t B, T, S_max, H_I, d_I;
} ix_indexer_args;

/* Precision of the per-kept-pair gradient rows that the atomic-free backward forms
 * (sparse_attn_bwd and ix_indexer_bwd with a workspace, indexshare_group_bwd) write and then
 * sum per key in fp32.  Not from the pages: an implementation choice.  BF16 rounds each row
 * once (relative error at most 2^-9 per element) and halves the rows' workspace and traffic;
 * FP32 stores the rows as the matrix cores left them, so the key sums round as the atomic
 * form's do, and stay bitwise reproducible. */
typedef enum ix_pair_rows { IX_PAIR_ROWS_BF16 = 0, IX_PAIR_ROWS_FP32 = 1 } ix_pair_rows;

/* ABI version of this header (bumped on any incompatible change). */
#define IX_ABI_VERSION 5
int32_t ix_abi_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char *ix_last_error(void);

/*
 * ix_score -- indexer scores (Stage 1) for query rows [t_begin, t_end).
 * scores: fp32 [B, t_end - t_begin, S_max]; entry (b, i, s) is the score of key s
 * for query t_begin + i, or -inf where s is not visible.  Written for every s.
 * This materialises score rows and exists to check Stage 1 on its own; ix_topk never
 * writes the T x S score matrix.
 * Errors: IX_ERR_INVALID for null pointers, negative dims or
 * 0 <= t_begin <= t_end <= T violated.
 */
ix_status ix_score(const ix_indexer_args *a, int32_t t_begin, int32_t t_end, float *scores,
                   hipStream_t stream);

/* Workspace bytes ix_topk needs for these arguments (0 on invalid arguments). */
size_t ix_topk_workspace_bytes(const ix_indexer_args *a, int32_t k);

/*
 * ix_topk -- Stage 1 + Stage 2 fused: per query, the min(k, n_t) visible keys with
 * the largest scores, ties broken towards the lower key index ("DeepSeek Sparse
 * Attention", Stage 2: fine selection).  Scores are streamed through the selection
 * and never written to memory.
 * idx:        int32 [B, T, k]: kept key positions in ascending order, then -1.
 * sel_scores: nullable fp32 [B, T, k]: the score of each kept key, -inf at padding.
 * ws:         device workspace of at least ix_topk_workspace_bytes(a, k) bytes
 *             (contents need no initialisation; clobbered).
 */
ix_status ix_topk(const ix_indexer_args *a, int32_t k, int32_t *idx, float *sel_scores,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes sparse_attn_fwd needs (0 on invalid arguments; may be 0). */
size_t sparse_attn_workspace_bytes(int32_t B, int32_t T, int32_t H_q, int32_t H_kv, int32_t d,
                                   int32_t k);

/*
 * sparse_attn_fwd -- softmax attention of each query over only its selected K/V
 * rows ("DeepSeek Sparse Attention", Stage 2: the kept tokens get full attention).
 * q:   bf16 [B, T, H_q, d];  kc, vc: bf16 caches [B, S_max, H_kv, d];
 * idx: int32 [B, T, k] key positions; entries < 0, >= S_max or >= kv_len[b] are
 *      skipped (padding).  Query head h reads KV head h / (H_q / H_kv).
 * kv_len: nullable device int32 [B] (NULL: S_max for every sequence).
 * out: bf16 [B, T, H_q, d] (round to nearest even).
 * lse: nullable fp32 [B, T, H_q], natural-log sum of exp of the scaled logits
 *      (-inf, with out = 0, when a query has no valid entry).
 * logits are sm_scale * q . k.
 */
ix_status sparse_attn_fwd(const void *q, const void *kc, const void *vc, const int32_t *idx,
                          const int32_t *kv_len, int32_t B, int32_t T, int32_t S_max,
                          int32_t H_q, int32_t H_kv, int32_t d, int32_t k, float sm_scale,
                          void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * sparse_attn_bwd -- gradients of sparse_attn_fwd over the same selection (the training
 * side: the twiscan post has the indexer learn from the attention distribution; these
 * are the attention's own gradients).  With p = softmax(sm_scale q K_J^T) per query head
 * (J the valid entries of idx) and D = dout . out:
 *   dq = sm_scale sum_j p_j (dout . V_j - D) K_j,
 *   dK_j += sm_scale p_j (dout . V_j - D) q,  dV_j += p_j dout  (summed over heads and
 *   over every query that selected row j).
 * q, kc, vc, idx, kv_len, B..sm_scale: as passed to sparse_attn_fwd; out and lse: its
 * outputs for these inputs (lse is required); dout: bf16 [B, T, H_q, d].
 * dq:       fp32 [B, T, H_q, d], written (0 for a query with no valid entry).
 * dkc, dvc: fp32 [B, S_max, H_kv, d], ADDED TO; the caller clears them first.  With
 *           atomics the order of the additions, and so the last bits, vary from run to run.
 *           The atomic-free form adds each key's pairs in query-row order: for a given
 *           workspace size (which sets the passes) the result is bitwise the same every run,
 *           except that the entries of one row that repeat a key may add in either order.
 * pair_rows: an ix_pair_rows value, the precision of the atomic-free form's pair rows
 *           (checked, and unused, without a workspace).
 * ws, ws_bytes: NULL and 0 -> dK / dV rows are added with fp32 atomics, 2 d per selected
 *           pair.  A workspace (16-byte aligned, at least sparse_attn_bwd_workspace_bytes(...,
 *           1, pair_rows) bytes, contents clobbered) -> no atomics: the query rows are taken
 *           in passes of as many rows as the workspace holds; each pass inverts the selection
 *           (pairs listed per key), writes every pair's dV and dK rows (in bf16 or fp32), and
 *           sums them per key in fp32.
 * Errors: as sparse_attn_fwd, plus IX_ERR_INVALID for NULL lse, dout or gradients, for
 * out/dout not 16-byte aligned, for lse or a gradient not 4-byte aligned, for another
 * pair_rows or for a misaligned workspace; IX_ERR_WORKSPACE for a workspace below one row's
 * need, or ws_bytes without a workspace.
 */
ix_status sparse_attn_bwd(const void *q, const void *kc, const void *vc, const int32_t *idx,
                          const int32_t *kv_len, const void *out, const float *lse,
                          const void *dout, int32_t B, int32_t T, int32_t S_max, int32_t H_q,
                          int32_t H_kv, int32_t d, int32_t k, float sm_scale, float *dq,
                          float *dkc, float *dvc, int32_t pair_rows, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* Workspace bytes for sparse_attn_bwd's atomic-free form in passes of rows_per_pass query
 * rows (clamped to B * T) with pair rows of precision pair_rows: the per-key offsets and
 * cursors (B * S_max + 1 each), the inverted selection (4 bytes per pair) and the pairs'
 * dV | dK rows (4 d H_kv bytes per pair in bf16, 8 d H_kv in fp32).  0 on invalid
 * arguments. */
size_t sparse_attn_bwd_workspace_bytes(int32_t B, int32_t T, int32_t S_max, int32_t H_kv,
                                       int32_t d, int32_t k, int32_t rows_per_pass,
                                       int32_t pair_rows);

/*
 * indexshare_group_bwd -- the attention backward of the n_layers layers of an IndexShare
 * group, which all attend over the same selection idx ("IndexShare: Amortizing the
 * Indexer" shares the selection; here its inversion is shared too): the atomic-free form of
 * sparse_attn_bwd in which, per pass over the query rows, the selection is inverted once
 * and every layer's dV | dK rows are summed per key through that inversion.  Layer l gets
 * what sparse_attn_bwd with a workspace gives for q[l], kc[l], ... (dq bit for bit; dK and
 * dV up to the order of the per-key sums).
 * q, kc, vc, out, lse, dout, dq, dkc, dvc: HOST arrays of n_layers device pointers, each as in
 *          sparse_attn_bwd (dkc[l], dvc[l] ADDED TO; the caller clears them first).
 * idx, kv_len, B..sm_scale, pair_rows: shared by the layers, as in sparse_attn_bwd.
 * ws:      required: at least sparse_attn_bwd_workspace_bytes(..., 1, pair_rows) bytes,
 *          16-byte aligned; the same layout and pass size as sparse_attn_bwd.
 * Errors: as sparse_attn_bwd for every layer, plus IX_ERR_INVALID for n_layers < 1 or a NULL
 * pointer array, IX_ERR_WORKSPACE without a workspace.
 */
ix_status indexshare_group_bwd(const int32_t *idx, const int32_t *kv_len, int32_t n_layers,
                               const void *const *q, const void *const *kc, const void *const *vc,
                               const void *const *out, const float *const *lse,
                               const void *const *dout, int32_t B, int32_t T, int32_t S_max,
                               int32_t H_q, int32_t H_kv, int32_t d, int32_t k, float sm_scale,
                               float *const *dq, float *const *dkc, float *const *dvc,
                               int32_t pair_rows, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * ix_indexer_kl -- the indexer's training objective (the twiscan post on GLM-5.2's
 * IndexShare: the indexer is trained to imitate the attention distribution with a KL
 * loss).  The page names the loss only; the reading implemented: for each query and the
 * valid entries j of its selection (0 <= idx < kv_len),
 *   u_j = sum over all H_q heads of exp(sm_scale q_h . K_j - lse_h),  t = u / sum_j u_j,
 *   pred = softmax_j(sel_scores_j),
 *   loss = sum_j t_j (log t_j - log pred_j),  dscores_j = pred_j - t_j.
 * With lse from sparse_attn_fwd over the same selection, t is the mean of the heads'
 * attention distributions; with a dense lse (every visible key), t is the dense
 * distribution restricted to the kept keys and renormalised.
 * q, kc, idx, kv_len, B..sm_scale: as passed to sparse_attn_fwd (vc is not needed).
 * lse:        fp32 [B, T, H_q] natural-log normalisers of the attention heads.
 * sel_scores: fp32 [B, T, k] indexer scores of the entries (ix_topk's sel_scores).
 * loss:       fp32 [B, T], written (0 for a query with no valid entry).
 * dscores:    fp32 [B, T, k], written: d loss / d sel_scores, 0 at padding.
 * Errors: as sparse_attn_fwd, plus IX_ERR_INVALID for NULL lse, sel_scores, loss or
 * dscores.
 */
ix_status ix_indexer_kl(const void *q, const void *kc, const int32_t *idx, const int32_t *kv_len,
                        const float *lse, const float *sel_scores, int32_t B, int32_t T,
                        int32_t S_max, int32_t H_q, int32_t H_kv, int32_t d, int32_t k,
                        float sm_scale, float *loss, float *dscores, hipStream_t stream);

/*
 * ix_indexer_bwd -- the KL objective's score gradient carried back into the indexer's own
 * inputs (the twiscan post on GLM-5.2's IndexShare: the indexer learns from the attention
 * distribution through a KL loss; the chain rule of the Stage-1 score form of "DeepSeek
 * Sparse Attention").  For each query, with x_hj = q_I[h,:] . k_I[s_j,:] over the valid
 * entries s_j of its selection (0 <= idx < min(kv_len, S_max)) and g_j = dscores:
 *   dw[h]      = sum_j g_j max(0, x_hj)
 *   dq_I[h,:]  = sum_j g_j w[h] [x_hj > 0] k_I[s_j,:]
 *   dk_I[s_j,:] += sum_h g_j w[h] [x_hj > 0] q_I[h,:]
 * Gradients are with respect to the decoded e4m3 values; the ReLU's step at x = 0 gets
 * gradient 0, and the mask [x > 0] is decided exactly.
 * a:       the indexer inputs of the forward, validated as for ix_topk (q_pos0 must be a
 *          valid pointer but is not read: idx says what is kept).
 * idx:     int32 [B, T, k] (ix_topk's output or any selection; invalid entries are skipped).
 * dscores: fp32 [B, T, k] (ix_indexer_kl's dscores); ignored at invalid entries.
 * dq_I:    fp32 [B, T, H_I, d_I], written.   dw: fp32 [B, T, H_I], written.
 * dk_I:    fp32 [B, S_max, d_I], ADDED TO; the caller clears it first.  With atomics the
 *          order of the additions, and so the last bits, vary from run to run; the
 *          atomic-free form is bitwise reproducible as for sparse_attn_bwd.
 * pair_rows: an ix_pair_rows value, the precision of the atomic-free form's dk_I rows
 *          (checked, and unused, without a workspace).
 * ws, ws_bytes: NULL and 0 -> dk_I rows are added with fp32 atomics, d_I per kept pair.  A
 *          workspace (16-byte aligned, at least ix_indexer_bwd_workspace_bytes(a, k, 1,
 *          pair_rows) bytes, contents clobbered) -> no atomics: passes of as many query rows
 *          as it holds, each inverting the selection, writing every pair's dk_I row (bf16 or
 *          fp32) and summing them per key in fp32 (as sparse_attn_bwd).
 * Errors: as ix_topk for the indexer arguments and k, plus IX_ERR_INVALID for NULL idx,
 * dscores or gradients, for w, idx, dscores or a gradient not 4-byte aligned, for another
 * pair_rows or for a misaligned workspace; IX_ERR_WORKSPACE for a workspace below one row's
 * need, or ws_bytes without a workspace.
 */
ix_status ix_indexer_bwd(const ix_indexer_args *a, int32_t k, const int32_t *idx,
                         const float *dscores, float *dq_I, float *dw, float *dk_I,
                         int32_t pair_rows, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for ix_indexer_bwd's atomic-free form in passes of rows_per_pass query
 * rows (clamped to B * T) with dk_I rows of precision pair_rows: per-key offsets and cursors
 * (B * S_max + 1 each), the inverted selection (4 bytes per pair) and the pairs' dk_I rows
 * (2 d_I bytes per pair in bf16, 4 d_I in fp32).  0 on invalid arguments. */
size_t ix_indexer_bwd_workspace_bytes(const ix_indexer_args *a, int32_t k, int32_t rows_per_pass,
                                      int32_t pair_rows);

/* Workspace bytes sparse_attn_group_fwd needs for n_layers layers (0 on invalid arguments;
 * may be 0): the split partials of the layers that share one launch. */
size_t sparse_attn_group_workspace_bytes(int32_t B, int32_t T, int32_t H_q, int32_t H_kv,
                                         int32_t d, int32_t k, int32_t n_layers);

/*
 * sparse_attn_group_fwd -- the attention of the n_layers layers of an IndexShare group over
 * one selection (the layers reuse one index tensor: "IndexShare: Amortizing the Indexer"),
 * with the selection computed by the caller (ix_topk, ix_topk_pooled or any other): layer l
 * gets what sparse_attn_fwd gives for q[l], kc[l], vc[l], out[l], lse[l] and the shared idx.
 * When one layer's grid is small (decode: B * T * H_kv < 1024 query rows) up to 8 layers
 * share one launch of the kernel made for few query rows that sparse_attn_fwd also uses
 * there (16-row chunks, K rows loaded straight into the matrix-core operands), and each
 * selection is split over as many blocks as make the launch about one block per CU, so over
 * fewer blocks than in a single-layer call; a layer's output then equals sparse_attn_fwd's up
 * to the rounding of P to bf16 against other running maxima and of the merge of the splits.
 * With 1024 query rows or more each layer runs as sparse_attn_fwd does, bit for bit.
 * q, kc, vc, out: HOST arrays of n_layers device pointers (shapes as in sparse_attn_fwd).
 * lse: nullable host array of n_layers nullable device pointers.
 * idx, kv_len, B..sm_scale: shared by the layers, as in sparse_attn_fwd.
 * ws: at least sparse_attn_group_workspace_bytes(B, T, H_q, H_kv, d, k, n_layers) bytes
 *     (NULL when that is 0; contents need no initialisation).
 * Errors: as sparse_attn_fwd for every layer, plus IX_ERR_INVALID for n_layers < 1 or a NULL
 * pointer array.
 */
ix_status sparse_attn_group_fwd(int32_t n_layers, const void *const *q, const void *const *kc,
                                const void *const *vc, void *const *out, float *const *lse,
                                const int32_t *idx, const int32_t *kv_len, int32_t B, int32_t T,
                                int32_t S_max, int32_t H_q, int32_t H_kv, int32_t d, int32_t k,
                                float sm_scale, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes indexshare_group_fwd needs, for any n_layers: the selection's, or the
 * split partials of the attention of the layers that share one launch. */
size_t indexshare_workspace_bytes(const ix_indexer_args *a, int32_t k, int32_t H_q,
                                  int32_t H_kv, int32_t d);

/*
 * indexshare_group_fwd -- IndexShare over a group of n_layers sparse layers: the
 * selection is computed once from the group's indexer inputs and every layer
 * attends over that same index tensor ("IndexShare: Amortizing the Indexer";
 * group of 4 in the pages).  Equivalent to ix_topk(a, k, idx) followed by
 * sparse_attn_group_fwd over the n_layers layers with the shared idx, bit for bit
 * (and so to sparse_attn_fwd per layer up to the rounding of split merges).
 * q, kc, vc, out: HOST arrays of n_layers device pointers (shapes as in
 *                 sparse_attn_fwd; kc/vc use S_max = a->S_max, kv_len = a->kv_len).
 * lse:            nullable host array of n_layers nullable device pointers.
 * idx:            caller-owned int32 [B, T, k]: written once, read n_layers times.
 * When one layer's attention grid is small (decode), the attention of up to 8 layers
 * runs in one launch (as sparse_attn_group_fwd).
 * ws_bytes: at least indexshare_workspace_bytes (less is accepted while it covers the
 * selection and sparse_attn_group_workspace_bytes for n_layers).
 */
ix_status indexshare_group_fwd(const ix_indexer_args *a, int32_t k, int32_t n_layers,
                               const void *const *q, const void *const *kc,
                               const void *const *vc, void *const *out, float *const *lse,
                               int32_t H_q, int32_t H_kv, int32_t d, float sm_scale,
                               int32_t *idx, void *ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the library's own scratch for indexshare_group_fwd_noalloc (64 MiB per GPU). */
#define IX_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * indexshare_group_fwd_noalloc -- indexshare_group_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same validation, kernels and results (bit for bit), but the workspace is
 * a scratch array inside the library, IX_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the
 * library runs on holds from the first call on it until the process ends.  The call
 * allocates nothing.  The caller still passes inputs and outputs (idx included).
 * Sizes: the call needs indexshare_workspace_bytes(a, k, H_q, H_kv, d) <= the scratch
 * (a decode step of up to about 128 sequences at 128K keys with top-2048 fits); larger
 * calls return IX_ERR_WORKSPACE before launching anything.
 * Concurrency: every call on one GPU uses that GPU's one scratch array, so calls that
 * overlap on one GPU (on different streams, or from different threads) race and give
 * undefined results; calls on one stream, or serialised by the caller, are safe.  Nothing
 * in the scratch needs to be cleared between calls.
 * Errors: as indexshare_group_fwd; IX_ERR_HIP also if the scratch's device address cannot
 * be found (first call on a device).
 */
ix_status indexshare_group_fwd_noalloc(const ix_indexer_args *a, int32_t k, int32_t n_layers,
                                       const void *const *q, const void *const *kc,
                                       const void *const *vc, void *const *out,
                                       float *const *lse, int32_t H_q, int32_t H_kv, int32_t d,
                                       float sm_scale, int32_t *idx, hipStream_t stream);

/*
 * IndexPool: pooling four indexer keys into one to cut long-context indexing cost
 * (GLM-5.3-Flash as recorded on worldresearchstate.com, "What changed").  The page says
 * no more; the reading implemented: a block key is the mean of `pool` consecutive
 * tokens' FP8 indexer keys rounded to e4m3 (tokens at or past kv_len count as zero), the
 * fused indexer + top-k scores blocks exactly as it scores keys, a query at position p
 * sees block j once pool*j <= p, and each kept block expands to its token positions.
 *
 * ix_pool_keys -- k_pooled [B, ceil(S_max/pool), d_I] e4m3 from k_I [B, S_max, d_I]
 * (both 8-byte aligned); kv_len: nullable device int32 [B] (NULL: S_max).
 * pool in {1, 2, 4, 8, 16} (a power of two keeps the mean exact before rounding).
 */
ix_status ix_pool_keys(const uint8_t *k_I, const int32_t *kv_len, int32_t B, int32_t S_max,
                       int32_t d_I, int32_t pool, uint8_t *k_pooled, hipStream_t stream);

/* Workspace bytes ix_topk_pooled needs (0 on invalid arguments). */
size_t ix_topk_pooled_workspace_bytes(const ix_indexer_args *a, int32_t pool, int32_t k_blocks);

/*
 * ix_topk_pooled -- Stage 1 + Stage 2 over block keys: per query the min(k_blocks,
 * visible blocks) best blocks (ties to the lower block), each expanded to its `pool`
 * token positions.
 * a:   as for ix_topk except that a->k points to the block keys [B, ceil(S_max/pool), d_I]
 *      (from ix_pool_keys); a->S_max, a->q_pos0 and a->kv_len count token positions.
 * idx: int32 [B, T, k_blocks * pool]: token positions in ascending order, then -1 (a kept
 *      block's tokens the query does not see are -1; only the last kept block can have
 *      them).
 * ws:  at least ix_topk_pooled_workspace_bytes(a, pool, k_blocks) bytes.
 * Errors as ix_topk; IX_ERR_UNSUPPORTED for pool outside {1, 2, 4, 8, 16} or k_blocks
 * outside 1..2048.
 */
ix_status ix_topk_pooled(const ix_indexer_args *a, int32_t pool, int32_t k_blocks, int32_t *idx,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * ix_append_kv -- the producer side of the caches, the step just before Stage 1 in a
 * decode loop: appends T_new tokens per sequence at positions pos0[b] + t.  New indexer
 * keys are rounded to FP8 e4m3 for the cache the FP8 indexer reads (the twiscan post on
 * GLM-5.2's IndexShare: the indexer runs in FP8): clamped to +-448, then rounded to the
 * nearest e4m3 value, ties to even (NaN stays NaN).  New K/V rows are copied as they are.
 * k_I_new:   fp32 [B, T_new, d_I] (16-byte aligned), or NULL to skip the indexer keys.
 * K_new, V_new: bf16 [B, T_new, H_kv, d] (16-byte aligned), each may be NULL to skip it.
 * pos0:      device int32 [B]; a token whose position falls outside [0, S_max) is skipped.
 * k_I_cache: [B, S_max, d_I] u8 (8-byte aligned); K_cache, V_cache: bf16 [B, S_max, H_kv, d].
 * A cache pointer must be given exactly when its new rows are.  kv_len stays the
 * caller's: the call writes cache rows only.
 * Errors: IX_ERR_INVALID for negative sizes, unpaired or misaligned pointers, a NULL pos0;
 * IX_ERR_UNSUPPORTED for d_I or d outside {64, 128} or H_kv outside 1..16.
 */
ix_status ix_append_kv(const float *k_I_new, const void *K_new, const void *V_new,
                       const int32_t *pos0, int32_t B, int32_t T_new, int32_t S_max, int32_t d_I,
                       int32_t H_kv, int32_t d, uint8_t *k_I_cache, void *K_cache, void *V_cache,
                       hipStream_t stream);

/*
 * Debug status -- not from the pages: a way to see, without a trap, what the kernels do
 * quietly.  Off by default.  While on (process-wide, from the next call), the library counts
 * into a status block that each GPU holds until the process ends:
 *   idx_out_of_range:      entries of a selection passed in by the caller that name no key,
 *                          i.e. lie outside [-1, kv_len) (-1 is the padding value); the
 *                          kernels skip such entries.  Each call that takes a selection
 *                          (sparse_attn_fwd, sparse_attn_group_fwd, sparse_attn_bwd,
 *                          indexshare_group_bwd, ix_indexer_kl, ix_indexer_bwd) counts each
 *                          such entry once, with one extra pass over idx;
 *   topk_compactions:      candidate buffers of the top-k that filled and were compacted in
 *                          place (a normal event; many of them mean a poor starting threshold);
 *   topk_resweeps:         top-k sweeps restarted from zero because the sampled starting
 *                          threshold kept too few keys (normal, and rare);
 *   topk_split_recomputes: queries whose key-split merge could not prove it held the top-k
 *                          and that were selected again without splits (normal);
 *   topk_overflow:         candidate entries dropped because a buffer had no room.  The
 *                          buffers are sized so that this cannot happen; the kernel skips
 *                          such a write rather than trapping, and a nonzero count means a
 *                          wrong selection.
 * Counting adds device-scope atomics and a pass over idx; the results are the same either
 * way.  Calls that overlap on one GPU add into the same block.
 */
typedef struct ix_debug_status {
  uint64_t idx_out_of_range;
  uint64_t topk_compactions;
  uint64_t topk_resweeps;
  uint64_t topk_split_recomputes;
  uint64_t topk_overflow;
} ix_debug_status;

/* Turns the debug status on (on = 1) or off (on = 0) for the calls that follow.
 * Errors: IX_ERR_INVALID for another value of on. */
ix_status ix_debug_enable(int32_t on);

/* Copies the debug status block of the stream's GPU to *status once the work queued on
 * `stream` has finished (the call synchronizes the stream), then, with reset != 0, zeroes
 * the block.  Errors: IX_ERR_INVALID for a NULL status; IX_ERR_HIP if the copy fails. */
ix_status ix_debug_read(ix_debug_status *status, int32_t reset, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* IX_H */
