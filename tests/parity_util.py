"""Acceptance checks shared by the GPU parity tests (HIP path vs the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from indexed_sparse_attention_ix_amd import synth
from oracle import ix_oracle as O

# tolerances
SCORE_RTOL = 1e-2          # indexer scores, relative
# plus the accumulation bound: each head's FP8 MFMA dot product is within FP8_MFMA_REL of
# sum_c |q_hc k_c|, and the H_I weighted heads are summed in fp32, so
# |err| <= (FP8_MFMA_REL + (H_I + 2) 2^-24) sum_h w_h sum_c |q_hc k_c|.  It only matters where
# the exact score is at (or next to) zero, e.g. a head whose dot product cancels exactly;
# there a relative bound cannot hold.
FP32_U = 2.0 ** -24
INDEX_BAND = 1e-3          # swaps allowed among keys within this relative band of the k-th score
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3
ATTN_ROW_REL = 2e-2        # per (row, head) ||o - o_ref||_2 / ||o_ref||_2
LSE_ABS = 2e-3
# MFMA dot products of exact products, error relative to the sum of the products' magnitudes
# (both asserted with a factor-2 margin by test_gpu_mfma_error.py):
FP8_MFMA_REL = 2.0 ** -10  # FP8 e4m3 16x16x128: its accumulation loses low bits of products of
                           # mixed sign (measured up to 2.8e-4 on codes spanning the whole range)
BF16_MFMA_REL = 2.0 ** -19  # bf16 16x16x32: accurate to about one fp32 rounding (8.6e-8 measured)
FP8_MASK_WINDOW = 2.0 ** -10  # the indexer backward recomputes exactly every x within this times
                              # |q|_2 |k|_2 of zero, so FP8 MFMA errors must stay below it
G_SPLIT_REL = 2.0 ** -16   # g as a hi + lo pair of bf16 (round to nearest twice): residual


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_host_indexer(ind):
    return {k: v.detach().cpu().numpy() for k, v in ind.items()}


def to_host_attn(att):
    return {k: synth.bf16_bits(v) for k, v in att.items()}


def score_magnitude(qI_row_u8, keys_abs, w_row):
    """sum_h |w_h| sum_c |q_hc| |k_sc| for every key row of keys_abs (fp64, [n, d_I])."""
    qa = np.abs(O.decode_e4m3(qI_row_u8))
    return np.abs(np.asarray(w_row, np.float64)) @ (qa @ keys_abs.T)


def score_tolerance(ref, mag, d_I, H_I):
    return SCORE_RTOL * np.abs(ref) + (FP8_MFMA_REL + (H_I + 2) * FP32_U) * mag


def check_scores(gpu_rows: np.ndarray, ref_rows: np.ndarray, mag_rows: np.ndarray, d_I, H_I):
    """gpu_rows, ref_rows, mag_rows: [R, S] (ref fp64, -inf where not visible)."""
    masked = np.isneginf(ref_rows)
    assert np.array_equal(np.isneginf(gpu_rows), masked), "visibility mask differs"
    g = gpu_rows[~masked].astype(np.float64)
    r = ref_rows[~masked]
    err = np.abs(g - r)
    bad = err > score_tolerance(r, mag_rows[~masked], d_I, H_I)
    assert not bad.any(), (f"{bad.sum()} scores outside tolerance; e.g. gpu {g[bad][:4]} "
                           f"ref {r[bad][:4]}")


def check_index_row(gpu_row: np.ndarray, ref_scores: np.ndarray, k: int, n_t: int, where=""):
    """Selection acceptance for one query.

    Structure: ascending distinct positions < n_t, exactly min(k, n_t) of them, then -1.
    Set: equal to the oracle's set except for swaps among keys whose oracle score lies
    within INDEX_BAND (relative) of the oracle's k-th score (when that score is 0 the band
    is {0}); the number of keys swapped in equals the number swapped out.
    """
    m = min(k, n_t)
    g = gpu_row[:m]
    assert np.all(gpu_row[m:] == -1), f"{where}: padding"
    assert np.all(g >= 0) and np.all(g < n_t), f"{where}: out of visible range"
    assert np.all(np.diff(g) > 0), f"{where}: not ascending/distinct"
    ref = O.select_topk(ref_scores, k)[:m]
    sg, so = set(g.tolist()), set(ref.tolist())
    d_in, d_out = sg - so, so - sg
    assert len(d_in) == len(d_out), f"{where}: swap counts differ"
    if d_in:
        sk = ref_scores[ref].min()
        for s in d_in | d_out:
            if sk == 0.0:
                assert ref_scores[s] == 0.0, f"{where}: key {s} outside the zero band"
            else:
                assert abs(ref_scores[s] - sk) <= INDEX_BAND * sk, (
                    f"{where}: key {s} score {ref_scores[s]} outside band of {sk}")
    return len(d_in)


def oracle_selection(gpu_rows: np.ndarray, ref_score_rows, k: int, n_ts, where=""):
    """Checks each GPU selection row against the oracle's scores (check_index_row) and
    returns (ref_idx [R, k], same [R]): the oracle's own selection, and the rows where the
    GPU kept exactly that set.  Values computed downstream of the selection (attention, KL,
    gradients) are compared on those rows, with the oracle working on its own selection; a
    row where the GPU kept another set that is equally valid (swaps inside the tie band)
    has been checked here and is left out there, so no GPU output ever enters the oracle."""
    ref = np.stack([O.select_topk(np.asarray(sc), k) for sc in ref_score_rows])
    same = np.zeros(len(ref), dtype=bool)
    for i, sc in enumerate(ref_score_rows):
        check_index_row(gpu_rows[i], np.asarray(sc), k, int(n_ts[i]), where=f"{where} row {i}")
        same[i] = np.array_equal(np.asarray(gpu_rows[i], dtype=np.int64), ref[i])
    return ref, same


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return O.decode_bf16(synth.bf16_bits(t))


def check_attention(out_gpu: np.ndarray, out_ref: np.ndarray, lse_gpu=None, lse_ref=None,
                    where=""):
    """out_*: [R, H, d] fp64 (GPU bf16 decoded)."""
    err = np.abs(out_gpu - out_ref)
    assert err.max() <= ATTN_MAX_ABS, f"{where}: max abs {err.max()}"
    assert err.mean() <= ATTN_MEAN_ABS, f"{where}: mean abs {err.mean()}"
    num = np.linalg.norm(out_gpu - out_ref, axis=-1)
    den = np.linalg.norm(out_ref, axis=-1)
    rel_ok = (num <= ATTN_ROW_REL * den) | ((den == 0) & (num == 0))
    assert rel_ok.all(), f"{where}: per-row relative error {np.max(num / np.maximum(den, 1e-30))}"
    if lse_gpu is not None:
        both_inf = np.isneginf(lse_gpu) & np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(lse_ref)), f"{where}: lse -inf"
        d = np.abs(lse_gpu[~both_inf] - lse_ref[~both_inf])
        assert d.size == 0 or d.max() <= LSE_ABS, f"{where}: lse err {d.max()}"


def abs_codes(c):
    return (np.asarray(c) & 0x7F).astype(np.uint8)


BF16_U = 2.0 ** -8         # bf16 keeps 8 significant bits: one round-to-nearest is within 2^-8


def attn_bwd_bounds(mags, k, n_rows, H_q, d, logit_mag, pair_rows):
    """Per-entry error bounds (dq, dK, dV) of sparse_attn_bwd, built from the oracle's sums of
    magnitudes (O.sparse_attention_backward_magnitudes: "ds" the row gradients |dl_j| =
    p_j |dp_j - D|, "dp" the size p_j a_j of dp's products, "dd"/"da" the shared D term).

    What the kernels round, and what each rounding can move:
      * P is recomputed in fp32 from the forward's lse: relative error eps_p <= 2.02 *
        logit_mag * BF16_MFMA_REL (the logits here and inside lse; logit_mag bounds
        sm_scale sum_c |q_c K_c|) plus fp32 roundings of the exponent, lse and exp2;
      * dp_j is an MFMA sum of exact bf16 products: off by BF16_MFMA_REL a_j;
      * D = dout . out uses the forward's bf16 output, off by (2 BF16_U + 2 eps_p) times
        sum_j p_j |V_jc| per entry, so D is off by cD A; the same error for every key of a
        (query, head), so in dq it multiplies |sum_j p_j K_j| ("dd"), not sum_j p_j |K_j|;
      * dS = P (dp - D) is rounded to bf16 (BF16_U) for the products with K (dq) and q (dK),
        which are MFMA sums (BF16_MFMA_REL) added in fp32 over keys, heads and queries (n 2^-24);
      * dV sums bf16-rounded P times dout;
      * the atomic-free form rounds each query's dK and dV pair row to bf16 (one more BF16_U).
    Every rounding is taken at its worst and in the same direction.
    """
    u = FP32_U
    eps_p = 2.02 * logit_mag * BF16_MFMA_REL + (k + 64 + 8 * logit_mag) * u
    f = (1 + eps_p) * (1 + BF16_U) * (1 + 4 * u)     # a computed P or dS over the exact one
    r = (eps_p + BF16_U) * (1 + eps_p) + 2 * u        # relative error of dS (or bf16 P)
    cD = 2 * BF16_U + 2 * eps_p + (d + 4) * u         # |D_gpu - D| / A
    g_q = BF16_MFMA_REL + (k + 64) * u                     # sums over the kept keys (dq)
    g_k = BF16_MFMA_REL + (n_rows * H_q + 64) * u          # sums over heads and queries (dK, dV)
    pair = BF16_U if pair_rows else 0.0
    mq, mk, mv = mags["dq"], mags["dK"], mags["dV"]
    sq = f * (mq["ds"] + BF16_MFMA_REL * mq["dp"] + cD * mq["da"])    # >= s sum_j |dS_gpu| |K_j|
    b_dq = r * mq["ds"] + f * (BF16_MFMA_REL * mq["dp"] + cD * (mq["dd"] + r * mq["da"])) + g_q * sq
    sk = f * (mk["ds"] + BF16_MFMA_REL * mk["dp"] + cD * mk["dd"])    # >= s sum |dS_gpu| |q|
    b_dK = r * mk["ds"] + f * (BF16_MFMA_REL * mk["dp"] + cD * mk["dd"]) + (g_k + pair * (1 + g_k)) * sk
    b_dV = r * mv["p"] + (g_k + pair * (1 + g_k)) * f * mv["p"]
    return b_dq, b_dK, b_dV


def logit_magnitude(q_f64, K_f64, sm_scale):
    """max over heads and keys of |sm_scale| sum_c |q_c| |K_c| (an upper bound through the
    largest |K| entry): q_f64 [..., H_q, d], K_f64 [..., d]."""
    qa = np.abs(q_f64).reshape(-1, q_f64.shape[-1]).sum(axis=1).max(initial=0.0)
    return abs(sm_scale) * float(qa) * float(np.abs(K_f64).max(initial=0.0))


def check_attn_bwd_entries(got, ref, bound, where="", power=None):
    """Every entry of got within bound of ref (an entry with bound 0 must be exact).
    power: also require that a wrong or missing row would be seen, i.e. that at least this
    fraction of the entries whose reference is not zero exceed their own bound (zeroing them
    would fail the check).  Returns the worst err / bound."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), (f"{where}: {int(bad.sum())} of {bad.size} entries out of tolerance; "
                           f"e.g. got {got[bad][:3]} ref {ref[bad][:3]} bound {bound[bad][:3]}")
    if power is not None:
        nz = ref != 0
        if nz.any():
            seen = float((np.abs(ref[nz]) > bound[nz]).mean())
            assert seen >= power, f"{where}: only {seen:.2f} of entries would show a missing row"
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, 0.0)
    return float(ratio.max()) if ratio.size else 0.0


def _indexer_bwd_oracle(qI, kI, w, idx, ds, kvl):
    """Oracle gradients and their magnitude bounds for every row of every sequence."""
    B, T = idx.shape[:2]
    out = []
    for b in range(B):
        rows = list(range(T))
        ref = O.indexer_backward_rows(qI, kI, w, idx[b], ds[b], b, rows, int(kvl[b]))
        mag = O.indexer_backward_rows(abs_codes(qI), abs_codes(kI), np.abs(w), idx[b],
                                      np.abs(ds[b]), b, rows, int(kvl[b]))
        out.append((ref, mag))
    return out


def indexer_bwd_coefficients(k, n_rows, bf16_rows=False):
    """Per-entry error bounds of ix_indexer_bwd relative to the oracle's gradients on absolute
    values (dq_I, dw, dk_I): dq_I and dk_I are bf16 MFMA products of g = dscores * w split into
    a hi + lo pair of bf16 (G_SPLIT_REL; two MFMAs) with exact e4m3 operands, summed over the
    kept keys (dq_I) or over heads and the queries keeping a key (dk_I) in fp32; dw sums
    g max(0, x) with x from the FP8 MFMA (FP8_MFMA_REL).  bf16_rows: the atomic-free form
    rounds each pair's dk_I row to bf16 (one more 2^-8)."""
    c_dq = G_SPLIT_REL + 2 * BF16_MFMA_REL + (64 + k) * FP32_U
    c_dw = FP8_MFMA_REL + (k + 2) * FP32_U
    c_dk = G_SPLIT_REL + 2 * BF16_MFMA_REL + (64 + n_rows) * FP32_U + (2.0 ** -8 if bf16_rows else 0.0)
    return c_dq, c_dw, c_dk


def check_indexer_bwd(got, qI, kI, w, idx, ds, kvl, extra=None, where="", bf16_rows=False):
    """ix_indexer_bwd outputs got = (dq_I, dw, dk_I) (host arrays) against the oracle, every
    entry, within the bound described in test_gpu_indexer_bwd.py: B = the oracle's gradient on
    absolute values, times indexer_bwd_coefficients.  extra: optional per-sequence
    additive bounds (dq, dw, dk) for errors that come in with dscores.  bf16_rows: dk_I came
    through per-pair rows rounded to bf16 (the atomic-free form): each term carries one more
    relative rounding of 2^-9, so dk_I's bound gains 2^-8 B."""
    dq, dw, dk = got
    B, T, k = idx.shape
    worst = [0.0, 0.0, 0.0]
    for b, (ref, mag) in enumerate(_indexer_bwd_oracle(qI, kI, w, idx, ds, kvl)):
        tols = indexer_bwd_coefficients(k, T, bf16_rows)
        for n, (g, r, m, tol) in enumerate(zip((dq[b], dw[b], dk[b]), ref, mag, tols)):
            bound = tol * m + (extra[b][n] if extra is not None else 0.0)
            err = np.abs(g.astype(np.float64) - r)
            name = ("dq_I", "dw", "dk_I")[n]
            bad = err > bound
            assert not bad.any(), (f"{where} {name} b={b}: {int(bad.sum())} entries out of tolerance; "
                                   f"max err {err.max():.3e}, e.g. got {g[bad][:3]} ref {r[bad][:3]}")
            with np.errstate(divide="ignore", invalid="ignore"):
                ratio = np.where(m > 0, err / m, 0.0)
            worst[n] = max(worst[n], float(ratio.max()) if ratio.size else 0.0)
    say(f"  worst err / magnitude: dq {worst[0]:.2e}  dw {worst[1]:.2e}  dk {worst[2]:.2e}")


def kl_tolerance(qf_row, Kf_seq, idx_row, scores_row, ref_dsc_row, sm_scale):
    """(loss bound, per-entry dscores bound) for ix_indexer_kl on one query.  The kernel forms
    the logits as fp32 sums of exact bf16 products, exponentiates and normalises in fp32:
    with logits of magnitude L the target and prediction carry relative errors of order
    1e-7 (1 + L), checked at eps = 2e-5 (1 + L): the loss within eps (plus 1e-5 of itself),
    each gradient entry pred_j - t_j within eps max(pred_j, t_j) + 1e-7.
    qf_row [H_q, d], Kf_seq [S, H_kv, d] (fp64), idx_row [k] (-1 where not valid)."""
    idx_row = np.asarray(idx_row)
    valid = idx_row >= 0
    bound = np.zeros(idx_row.shape)
    if not valid.any():
        return 0.0, bound
    v = idx_row[valid]
    L = float(np.abs(sm_scale * np.einsum("jgd,hd->jgh", Kf_seq[v], qf_row)).max())
    eps = 2e-5 * (1 + L)
    sc = np.asarray(scores_row, dtype=np.float64)[valid]
    e = np.exp(sc - sc.max())
    pred = e / e.sum()
    bound[valid] = eps * np.maximum(pred, np.abs(pred - np.asarray(ref_dsc_row)[valid])) + 1e-7
    return eps, bound
