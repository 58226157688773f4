"""CPU oracle for the indexer -> top-k -> sparse-attention path, in fp64.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package entry's smoke check and
the benchmark's CPU-baseline leg may import or run this module.  The HIP library never
calls it, links it or shares code with it, and this module imports nothing from the
library or its package (inputs reach it as plain numpy arrays).

It is the plain definition of what the path computes, written out with no blocking,
fusion or reordering:

  * Stage 1 (coarse scoring): an indexer scores every causal key for the current
    query ("GLM 5.2: How Four Co-Designed Mechanisms Beat Raw Scale", Part II,
    "DeepSeek Sparse Attention", Stage 1).  The indexer runs in FP8 (twiscan post on
    GLM-5.2's IndexShare).  Concrete form adopted: per indexer head h, the dot product
    of the FP8 query row q_I[t,h,:] with the FP8 key row k_I[s,:]; then ReLU; then
    the sum over heads weighted by w[t,h].
  * Stage 2 (fine selection): keep the k best-scoring keys (k = 2048 at full size;
    same page, Stage 2).  Ties go to the lower key index.  Output is the ascending
    list of kept positions padded with -1.
  * Attention over only the kept keys: ordinary softmax attention restricted to the
    selected rows (same page, Stage 2; the twiscan post).
  * IndexShare: the selection is computed once per group of 4 sparse layers and
    reused by the others (same page, "IndexShare: Amortizing the Indexer"; the
    twiscan post; "The 1M Context Mirage", "IndexShare: What Actually Works").
  * IndexPool (GLM-5.3-Flash, worldresearchstate.com record, "What changed": four
    indexer keys pooled into one to cut long-context indexing cost).  The page does not
    say how keys are pooled or how a pooled selection maps back to tokens; the reading
    here is the plainest one: a block key is the mean of 4 consecutive tokens' FP8
    indexer keys, rounded to e4m3 (a block cut short by kv_len counts its missing tokens
    as zero, so every block divides by 4 and the mean is exact before rounding); the indexer
    scores blocks exactly as it scores keys; a query at position p sees block j iff
    4j <= p; the best k/4 blocks are kept (ties to the lower block) and each expands to
    its tokens that the query sees, in ascending order, padded with -1.
  * Training side (the twiscan post: the indexer is trained to imitate the attention
    distribution with a KL loss): gradients of the sparse attention with respect to q, K
    and V, the plain chain rule through softmax over the selected rows; and the KL
    objective, read as: target t over the selected keys = the attention probabilities
    exp(l_hj - lse_h) summed over the query heads and normalised to sum 1 over the
    selection (lse_h defaults to the log-sum-exp over the selection itself, which makes
    t the mean of the heads' sparse distributions; a dense lse gives the dense
    distribution restricted to the kept keys), prediction = softmax of the indexer
    scores of the same keys, loss = KL(t || prediction), gradient with respect to the
    scores = prediction - t; and that gradient carried back into the indexer's inputs
    q_I, k_I and w by the chain rule through the head sum and the ReLU (gradient with
    respect to the decoded e4m3 values; the ReLU's step at 0 gets gradient 0).
  * Cache append (the step before Stage 1 in a decode loop): new indexer keys are
    rounded to FP8 e4m3 and written into the FP8 key cache, new K/V rows into theirs.
    The pages say only that the indexer runs in FP8 (twiscan post); the rounding read
    here is the plain one: clamp to the largest finite e4m3 magnitude (448), then round
    to the nearest e4m3 value, ties to the even code.

Exactness.  Every e4m3 value is an integer multiple of 2^-9 below 2^9 in magnitude, so
each product is a multiple of 2^-18 below 2^18 and any partial sum of at most 128 such
products needs at most 43 significant bits: the per-head dot products below are exact
in fp64 whatever order BLAS adds them in.  The only roundings are in w*x, the head sum
and the attention arithmetic (relative ~1e-16).

Readings where the pages are silent (all listed with their reasons in the design notes):
  visibility  key s is visible to the query at position p iff s <= p and s < kv_len
              (a query sees its own key); n_t = min(p + 1, kv_len).
  ties        lowest key index wins; fewer than k visible keys -> take all, pad -1.
  scale       the indexer score carries no extra scale factor.
  heads       one indexer key row per token, shared by all indexer heads;
              head weights are per (query token, indexer head).
  empty       an empty selection gives out = 0 and lse = -inf.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np

# ----------------------------------------------------------------------------------
# Storage formats
# ----------------------------------------------------------------------------------


def _e4m3_value(code: int) -> float:
    """OCP FP8 E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no
    infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """e4m3 bytes (uint8 array) -> exact fp64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """Values -> e4m3 bytes: clamp to [-448, 448], then round to nearest, ties to even.

    Constructive form of the OCP E4M3 grid: in the binade [2^E, 2^(E+1)) (E >= -6) the
    spacing is 2^(E-3); below 2^-6 (subnormals) it is 2^-9.  Dividing by the spacing,
    rounding half to even and multiplying back gives the rounded value exactly in fp64
    (a value that rounds up to 2^(E+1) is the next binade's first value).  The sign is
    kept (so -0 and values rounding to zero from below give the negative-zero code);
    NaN gives the NaN code S.1111.111.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    for i, v in enumerate(flat):
        sign = 0x80 if math.copysign(1.0, v) < 0 else 0
        if math.isnan(v):
            res[i] = sign | 0x7F
            continue
        a = min(abs(v), 448.0)
        if a < 2.0 ** -6:
            spacing = 2.0 ** -9
        else:
            spacing = 2.0 ** (math.floor(math.log2(a)) - 3)
        r = float(np.rint(a / spacing)) * spacing
        # the code of the rounded magnitude: exponent field and mantissa from r
        if r < 2.0 ** -6:
            code = int(round(r / 2.0 ** -9))           # subnormal: m/8 * 2^-6
        else:
            e = math.floor(math.log2(r))
            m = int(round((r / 2.0 ** e - 1.0) * 8))
            code = ((e + 7) << 3) | m
        res[i] = sign | code
    return out


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64: a bf16 is the upper half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------
# Stage 1: indexer scores
# ----------------------------------------------------------------------------------


def visible_count(pos0: int, kv_len: int, t: int) -> int:
    """Number of keys visible to query t of a sequence: keys [0, n_t)."""
    return max(0, min(int(pos0) + t + 1, int(kv_len)))


def index_scores(q_row: np.ndarray, keys: np.ndarray, w_row: np.ndarray) -> np.ndarray:
    """score[s] = sum_h w[h] * max(0, q[h,:] . k[s,:]) for the given key rows.

    q_row [H_I, d_I] fp64, keys [n, d_I] fp64, w_row [H_I] fp64 -> [n] fp64.
    (Stage 1 of "DeepSeek Sparse Attention" with the ReLU / weighted-head-sum form.)
    """
    x = q_row @ keys.T                    # [H_I, n]: per-head dot products (exact)
    return w_row @ np.maximum(x, 0.0)     # ReLU, then the w-weighted sum over heads


KEY_CHUNK = 1 << 17  # keys per call of index_scores (each key's score is independent)


def score_row(qI_row_u8, keys_f64, w_row, n_t) -> np.ndarray:
    """Scores of the n_t visible keys for one query (decoded keys given)."""
    q = decode_e4m3(qI_row_u8)
    w = np.asarray(w_row, dtype=np.float64)
    out = np.empty(n_t, dtype=np.float64)
    for s0 in range(0, n_t, KEY_CHUNK):
        s1 = min(n_t, s0 + KEY_CHUNK)
        out[s0:s1] = index_scores(q, keys_f64[s0:s1], w)
    return out


def score_matrix(q_I, k_I, w, q_pos0, kv_len, b: int, rows: Sequence[int], S_max: int):
    """Dense [len(rows), S_max] fp64 score rows for sequence b; -inf where not visible."""
    keys = decode_e4m3(k_I[b])
    out = np.full((len(rows), S_max), -np.inf, dtype=np.float64)
    for i, t in enumerate(rows):
        n = visible_count(q_pos0[b], kv_len[b], t)
        out[i, :n] = score_row(q_I[b, t], keys[:n], w[b, t], n)
    return out


# ----------------------------------------------------------------------------------
# Stage 2: top-k selection
# ----------------------------------------------------------------------------------


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Keep the first min(k, n) keys in (score descending, index ascending) order.

    Returns int64 [k]: the kept positions in ascending order, then -1 padding.
    """
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))  # primary -score, then index
    kept = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[: kept.shape[0]] = kept
    return out


def topk_rows(q_I, k_I, w, q_pos0, kv_len, b: int, rows: Sequence[int], k: int,
              keys_f64=None, return_scores=False):
    """Selection (and optionally the score rows) for the listed queries of sequence b."""
    keys = decode_e4m3(k_I[b]) if keys_f64 is None else keys_f64
    idx = np.empty((len(rows), k), dtype=np.int64)
    scores: List[np.ndarray] = []
    for i, t in enumerate(rows):
        n = visible_count(q_pos0[b], kv_len[b], t)
        sc = score_row(q_I[b, t], keys[:n], w[b, t], n)
        idx[i] = select_topk(sc, k)
        if return_scores:
            scores.append(sc)
    return (idx, scores) if return_scores else idx


# ----------------------------------------------------------------------------------
# Attention over the selected keys
# ----------------------------------------------------------------------------------


def sparse_attention_row(q_row, K_seq, V_seq, idx_row, sm_scale: float):
    """Softmax attention of one query token over its selected key rows.

    q_row [H_q, d] fp64; K_seq, V_seq [S, H_kv, d] fp64; idx_row [k] (-1 = padding).
    Query head h reads KV head h // (H_q / H_kv).  Returns out [H_q, d], lse [H_q].
    """
    H_q, d = q_row.shape
    H_kv = K_seq.shape[1]
    grp = H_q // H_kv
    sel = np.asarray(idx_row)[np.asarray(idx_row) >= 0]
    out = np.zeros((H_q, d), dtype=np.float64)
    lse = np.full(H_q, -np.inf, dtype=np.float64)
    if sel.size == 0:
        return out, lse
    for h in range(H_q):
        Kh = K_seq[sel, h // grp, :]          # gathered key rows [m, d]
        Vh = V_seq[sel, h // grp, :]
        logits = sm_scale * (Kh @ q_row[h])   # [m]
        mx = logits.max()
        p = np.exp(logits - mx)
        l = p.sum()
        out[h] = (p @ Vh) / l
        lse[h] = mx + math.log(l)
    return out, lse


def sparse_attention_rows(q_bits, K_bits, V_bits, idx, b: int, rows: Sequence[int],
                          sm_scale: float):
    """Attention outputs for the listed queries of sequence b (bf16 inputs as bits).

    idx is indexed like rows: idx[i] is the selection of query rows[i].
    Returns out [len(rows), H_q, d] and lse [len(rows), H_q], fp64.
    """
    K = decode_bf16(K_bits[b])
    V = decode_bf16(V_bits[b])
    H_q, d = q_bits.shape[2], q_bits.shape[3]
    out = np.empty((len(rows), H_q, d), dtype=np.float64)
    lse = np.empty((len(rows), H_q), dtype=np.float64)
    for i, t in enumerate(rows):
        q = decode_bf16(q_bits[b, t])
        out[i], lse[i] = sparse_attention_row(q, K, V, idx[i], sm_scale)
    return out, lse


def sparse_attention_backward_rows(q_bits, K_bits, V_bits, idx, dout, b: int,
                                   rows: Sequence[int], sm_scale: float):
    """Gradients of out = softmax(sm_scale * q K_sel^T) V_sel for the listed queries of
    sequence b, given dout [len(rows), H_q, d] (fp64).

    Per query head h with selected rows J: p = softmax(l), l_j = sm_scale q.K_j;
    dV_j += p_j dO;  dp_j = dO.V_j;  D = sum_j p_j dp_j (= dO.o);  dl_j = p_j (dp_j - D);
    dq = sm_scale sum_j dl_j K_j;  dK_j += sm_scale dl_j q.
    Returns dq [len(rows), H_q, d] and dK, dV [S, H_kv, d] (summed over the rows).
    """
    K = decode_bf16(K_bits[b])
    V = decode_bf16(V_bits[b])
    S, H_kv, d = K.shape
    H_q = q_bits.shape[2]
    grp = H_q // H_kv
    dq = np.zeros((len(rows), H_q, d), dtype=np.float64)
    dK = np.zeros((S, H_kv, d), dtype=np.float64)
    dV = np.zeros((S, H_kv, d), dtype=np.float64)
    for i, t in enumerate(rows):
        q = decode_bf16(q_bits[b, t])
        sel = np.asarray(idx[i])[np.asarray(idx[i]) >= 0]
        if sel.size == 0:
            continue
        for h in range(H_q):
            g = h // grp
            Kh, Vh = K[sel, g, :], V[sel, g, :]
            logits = sm_scale * (Kh @ q[h])
            p = np.exp(logits - logits.max())
            p /= p.sum()
            do = dout[i, h]
            dp = Vh @ do
            D = float(p @ dp)
            dl = p * (dp - D)
            dq[i, h] = sm_scale * (dl @ Kh)
            np.add.at(dK[:, g, :], sel, sm_scale * dl[:, None] * q[h][None, :])
            np.add.at(dV[:, g, :], sel, p[:, None] * do[None, :])
    return dq, dK, dV


def sparse_attention_backward_magnitudes(q_bits, K_bits, V_bits, idx, dout, b: int,
                                         rows: Sequence[int], sm_scale: float):
    """Sums of absolute values along the chain rule of sparse_attention_backward_rows, per
    gradient entry: the scales that rounding-error bounds of a computed backward are built
    from (they are not gradients).

    With p, dp_j = dO.V_j, D = sum_j p_j dp_j and dl_j = p_j (dp_j - D) as there, and
    a_j = sum_c |dO_c V_jc| (the size of dp_j's products), A = sum_j p_j a_j:
      dq[h, e]:  "ds" = s sum_j |dl_j| |K_je|     "dp" = s sum_j p_j a_j |K_je|
                 "dd" = s A |sum_j p_j K_je|      "da" = s A sum_j p_j |K_je|
      dK[j, e]:  "ds" = s sum |dl_j| |q_e|        "dp" = s sum p_j a_j |q_e|
                 "dd" = s sum p_j A |q_e|         (sums over the (query, head) pairs keeping j)
      dV[j, e]:  "p"  = sum p_j |dO_e|
    with s = |sm_scale|.  Returns {"dq": {...}, "dK": {...}, "dV": {...}} of arrays shaped as
    the corresponding gradients.
    """
    Ks = decode_bf16(K_bits[b])
    V = decode_bf16(V_bits[b])
    Ka, Va = np.abs(Ks), np.abs(V)
    S, H_kv, d = Ks.shape
    H_q = q_bits.shape[2]
    grp = H_q // H_kv
    s = abs(sm_scale)
    zq = lambda: np.zeros((len(rows), H_q, d), dtype=np.float64)  # noqa: E731
    zk = lambda: np.zeros((S, H_kv, d), dtype=np.float64)  # noqa: E731
    out = {"dq": {n: zq() for n in ("ds", "dp", "dd", "da")},
           "dK": {n: zk() for n in ("ds", "dp", "dd")}, "dV": {"p": zk()}}
    mq, mk, mv = out["dq"], out["dK"], out["dV"]
    for i, t in enumerate(rows):
        q = decode_bf16(q_bits[b, t])
        sel = np.asarray(idx[i])[np.asarray(idx[i]) >= 0]
        if sel.size == 0:
            continue
        for h in range(H_q):
            g = h // grp
            logits = sm_scale * (Ks[sel, g, :] @ q[h])
            p = np.exp(logits - logits.max())
            p /= p.sum()
            do = dout[i, h]
            dp = V[sel, g, :] @ do
            D = float(p @ dp)
            adl = np.abs(p * (dp - D))
            a = Va[sel, g, :] @ np.abs(do)
            A = float(p @ a)
            mq["ds"][i, h] = s * (adl @ Ka[sel, g, :])
            mq["dp"][i, h] = s * ((p * a) @ Ka[sel, g, :])
            mq["dd"][i, h] = s * A * np.abs(p @ Ks[sel, g, :])
            mq["da"][i, h] = s * A * (p @ Ka[sel, g, :])
            aq = np.abs(q[h])[None, :]
            np.add.at(mk["ds"][:, g, :], sel, s * adl[:, None] * aq)
            np.add.at(mk["dp"][:, g, :], sel, s * (p * a)[:, None] * aq)
            np.add.at(mk["dd"][:, g, :], sel, s * (p * A)[:, None] * aq)
            np.add.at(mv["p"][:, g, :], sel, p[:, None] * np.abs(do)[None, :])
    return out


def indexer_kl_rows(q_bits, K_bits, idx, scores, b: int, rows: Sequence[int], sm_scale: float,
                    kv_len: int, lse=None):
    """KL objective of the indexer for the listed queries of sequence b.

    idx [len(rows), k] selections (entries < 0 or >= kv_len are padding), scores
    [len(rows), k] the indexer's scores of those entries, lse optional [len(rows), H_q]
    natural-log normalisers of the attention heads.  Per query:
      u_j = sum_h exp(sm_scale q_h.K_j - lse_h),  t = u / sum(u),
      pred = softmax(scores over the kept entries),
      loss = sum_j t_j (log t_j - log pred_j),  dscores = pred - t (0 at padding).
    Returns loss [len(rows)] and dscores [len(rows), k]; an empty selection gives 0.
    """
    K = decode_bf16(K_bits[b])
    H_q = q_bits.shape[2]
    grp = H_q // K.shape[1]
    loss = np.zeros(len(rows), dtype=np.float64)
    dsc = np.zeros(np.asarray(scores).shape, dtype=np.float64)
    for i, t in enumerate(rows):
        q = decode_bf16(q_bits[b, t])
        row = np.asarray(idx[i])
        valid = (row >= 0) & (row < kv_len)
        if not valid.any():
            continue
        sel = row[valid]
        u = np.zeros(sel.size)
        for h in range(H_q):
            logits = sm_scale * (K[sel, h // grp, :] @ q[h])
            if lse is None:
                mx = logits.max()
                lse_h = mx + np.log(np.exp(logits - mx).sum())
            else:
                lse_h = float(lse[i][h])
            u += np.exp(logits - lse_h)
        target = u / u.sum()
        sc = np.asarray(scores[i], dtype=np.float64)[valid]
        mx = sc.max()
        log_pred = sc - mx - np.log(np.exp(sc - mx).sum())
        with np.errstate(divide="ignore", invalid="ignore"):
            terms = np.where(target > 0, target * (np.log(target) - log_pred), 0.0)
        loss[i] = terms.sum()
        dsc[i, valid] = np.exp(log_pred) - target
    return loss, dsc


def indexer_backward_rows(q_I, k_I, w, idx, dscores, b: int, rows: Sequence[int], kv_len: int):
    """Gradients of the kept keys' indexer scores with respect to the indexer's inputs,
    for the listed queries of sequence b, given g_j = d loss / d score_j (the KL's dscores).

    With x_hj = q_I[t,h,:] . k_I[s_j,:] and score_j = sum_h w[t,h] max(0, x_hj):
      dw[t,h]     = sum_j g_j max(0, x_hj)
      dq_I[t,h,:] = sum_j g_j w[t,h] [x_hj > 0] k_I[s_j,:]
      dk_I[s,:]   = sum over the listed (t, j) with s_j = s of sum_h g_j w[t,h] [x_hj > 0] q_I[t,h,:]
    Gradients are taken with respect to the decoded e4m3 values, and the ReLU's step at
    x = 0 gets gradient 0 (both readings; the pages give no more than the KL objective).
    idx [len(rows), k] (entries < 0 or >= min(kv_len, S_max) are padding), dscores
    [len(rows), k].  Returns dq [len(rows), H_I, d_I], dw [len(rows), H_I] and dk
    [S_max, d_I], the listed rows' share of the key gradient.  The dot products x are exact
    (see Exactness above), so the mask [x > 0] is the exact one.
    """
    keys = decode_e4m3(k_I[b])
    n_keys = min(int(kv_len), keys.shape[0])
    H_I, d_I = q_I.shape[2], q_I.shape[3]
    dq = np.zeros((len(rows), H_I, d_I), dtype=np.float64)
    dw = np.zeros((len(rows), H_I), dtype=np.float64)
    dk = np.zeros_like(keys)
    for i, t in enumerate(rows):
        row = np.asarray(idx[i])
        valid = (row >= 0) & (row < n_keys)
        if not valid.any():
            continue
        sel = row[valid]
        g = np.asarray(dscores[i], dtype=np.float64)[valid]
        q = decode_e4m3(q_I[b, t])                  # [H_I, d_I]
        wt = np.asarray(w[b, t], dtype=np.float64)  # [H_I]
        x = q @ keys[sel].T                         # [H_I, n], exact
        dw[i] = np.maximum(x, 0.0) @ g
        G = (x > 0) * wt[:, None] * g[None, :]     # d loss / d x
        dq[i] = G @ keys[sel]
        np.add.at(dk, sel, G.T @ q)
    return dq, dw, dk


# ----------------------------------------------------------------------------------
# IndexShare: one selection per group of layers
# ----------------------------------------------------------------------------------


def indexshare_group(indexer: Dict[str, np.ndarray], layers: Sequence[Dict[str, np.ndarray]],
                     k: int, b: int, rows: Sequence[int], sm_scale: float):
    """Selection computed once from the group's indexer inputs, reused by every layer.

    indexer: q_I, k_I, w, q_pos0, kv_len (numpy).  layers: per-layer q, K, V bits.
    Returns (idx [len(rows), k], [(out, lse) per layer]).
    """
    idx = topk_rows(indexer["q_I"], indexer["k_I"], indexer["w"], indexer["q_pos0"],
                    indexer["kv_len"], b, rows, k)
    outs = [sparse_attention_rows(L["q"], L["K"], L["V"], idx, b, rows, sm_scale)
            for L in layers]
    return idx, outs


# ----------------------------------------------------------------------------------
# Cache append: the producer side of the FP8 key cache and the K/V caches
# ----------------------------------------------------------------------------------


def append_kv(k_I_cache, K_cache, V_cache, k_I_new, K_new, V_new, pos0):
    """Copies of the caches after appending T_new tokens per sequence at pos0[b] + t.

    k_I_cache [B, S, d_I] uint8, K_cache/V_cache [B, S, H_kv, d] uint16 (bf16 bits) or
    None; k_I_new [B, T_new, d_I] float32 values, K_new/V_new [B, T_new, H_kv, d] bf16
    bits or None.  Positions outside [0, S) are skipped.
    """
    kc = None if k_I_cache is None else np.array(k_I_cache, copy=True)
    Kc = None if K_cache is None else np.array(K_cache, copy=True)
    Vc = None if V_cache is None else np.array(V_cache, copy=True)
    ref = kc if kc is not None else Kc
    B, S = ref.shape[0], ref.shape[1]
    new = k_I_new if k_I_new is not None else K_new
    T_new = new.shape[1]
    for b in range(B):
        for t in range(T_new):
            pos = int(pos0[b]) + t
            if pos < 0 or pos >= S:
                continue
            if kc is not None:
                kc[b, pos] = encode_e4m3(k_I_new[b, t])
            if Kc is not None:
                Kc[b, pos] = K_new[b, t]
            if Vc is not None:
                Vc[b, pos] = V_new[b, t]
    return kc, Kc, Vc


# ----------------------------------------------------------------------------------
# IndexPool: scoring blocks of pooled indexer keys
# ----------------------------------------------------------------------------------


def pool_keys(k_I_seq: np.ndarray, kv_len: int, pool: int) -> np.ndarray:
    """[S, d_I] e4m3 bytes of one sequence -> [ceil(S/pool), d_I] e4m3 bytes: the sum of
    each block's keys below kv_len divided by pool (the mean of a full block; missing
    tokens count as zero), rounded to e4m3."""
    S, d_I = k_I_seq.shape
    nb = (S + pool - 1) // pool
    vals = decode_e4m3(k_I_seq)
    out = np.zeros((nb, d_I), dtype=np.uint8)
    for j in range(nb):
        lo, hi = pool * j, min(pool * j + pool, S, max(kv_len, 0))
        if hi > lo:
            out[j] = encode_e4m3(vals[lo:hi].sum(axis=0) / pool)
    return out


def visible_blocks(pos0: int, kv_len: int, t: int, pool: int) -> int:
    """Blocks visible to query t: block j iff pool*j <= pos0 + t and pool*j < kv_len."""
    p = pos0 + t
    if p < 0:
        return 0
    return min(p // pool + 1, (max(kv_len, 0) + pool - 1) // pool)


def pooled_topk_row(qI_row, pooled_keys_f64, w_row, pos0, kv_len, t, pool, k_blocks):
    """(block scores over the visible blocks, kept blocks, expanded token row of length
    k_blocks * pool)."""
    nb = visible_blocks(pos0, kv_len, t, pool)
    sc = score_row(qI_row, pooled_keys_f64[:nb], w_row, nb)
    blocks = select_topk(sc, k_blocks)
    n_t = visible_count(pos0, kv_len, t)
    toks = [pool * j + r for j in blocks if j >= 0 for r in range(pool) if pool * j + r < n_t]
    row = np.full(k_blocks * pool, -1, dtype=np.int64)
    row[:len(toks)] = toks
    return sc, blocks, row
