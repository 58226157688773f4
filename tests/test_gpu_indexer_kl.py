"""GPU parity: the indexer's KL objective (ix_indexer_kl) against the oracle.

Tolerance.  The kernel forms the logits as fp32 sums of exact bf16 products (relative
error ~2^-24 sqrt(d) of sum |q_c K_c|), exponentiates in fp32 and normalises in fp32; with
logits of magnitude L the target and prediction carry relative errors of order
1e-7 (1 + L).  The loss is a sum of terms t_j (log t_j - log pred_j) with sum t_j = 1, so
its absolute error is of the same order: checked at 2e-5 (1 + L) plus 1e-5 |loss|.
Each gradient entry pred_j - t_j is checked at 2e-5 (1 + L) max(pred_j, t_j) + 1e-7.
"""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from oracle import ix_oracle as O
from parity_util import kl_tolerance, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _check(loss, dsc, idx, scores, q, K, kvl, scale, lse=None, rows_of=None):
    """Compare every row of loss/dsc with the oracle (lse: optional host [B,T,H_q])."""
    B, T = loss.shape
    qb, Kb = _bits(q), _bits(K)
    qf, Kf = q.float(), K.float()
    for b in range(B):
        ref_l, ref_d = O.indexer_kl_rows(qb, Kb, idx[b], scores[b], b, list(range(T)), scale,
                                         int(kvl[b]), lse=None if lse is None else lse[b])
        for t in range(T):
            v = idx[b, t][(idx[b, t] >= 0) & (idx[b, t] < kvl[b])]
            L = float((scale * (Kf[b, v, 0, :] @ qf[b, t].T)).abs().max()) if v.size else 0.0
            eps = 2e-5 * (1 + L)
            assert abs(loss[b, t] - ref_l[t]) <= eps + 1e-5 * abs(ref_l[t]), \
                f"loss b={b} t={t}: {loss[b, t]} vs {ref_l[t]}"
            sc = np.asarray(scores[b, t], dtype=np.float64)
            valid = (idx[b, t] >= 0) & (idx[b, t] < kvl[b])
            pred = np.zeros_like(sc)
            if valid.any():
                e = np.exp(sc[valid] - sc[valid].max())
                pred[valid] = e / e.sum()
            tgt = pred - ref_d[t]
            bound = eps * np.maximum(pred, np.abs(tgt)) + 1e-7
            err = np.abs(dsc[b, t] - ref_d[t])
            assert np.all(err <= bound), f"dscores b={b} t={t}: max err {err.max():.3e}"
            assert np.all(dsc[b, t][~valid] == 0)


def _random_case(B, T, S, H_q, H_kv, d, k, seed, kv_lens=None, sharp=1.0, empty_rows=()):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = (torch.randn(B, T, H_q, d, generator=g) * sharp * d ** -0.25).to(torch.bfloat16)
    K = (torch.randn(B, S, H_kv, d, generator=g) * d ** -0.25).to(torch.bfloat16)
    V = torch.randn(B, S, H_kv, d, generator=g).to(torch.bfloat16)
    kvl = np.array(kv_lens if kv_lens is not None else [S] * B, dtype=np.int32)
    rng = np.random.default_rng(seed)
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            if (b, t) in empty_rows:
                continue
            n = int(rng.integers(1, k + 1))
            idx[b, t, :n] = np.sort(rng.choice(S, size=n, replace=False))
    scores = (rng.standard_normal((B, T, k)) * 2).astype(np.float32)
    scores[idx < 0] = -np.inf
    return q, K, V, kvl, idx, scores


def _gpu_kl(q, K, V, kvl, idx, scores, scale, lse=None):
    dq, dK, dV = (x.to(DEV) for x in (q, K, V))
    didx = torch.from_numpy(idx).to(DEV)
    dkvl = torch.from_numpy(kvl).to(DEV)
    if lse is None:
        _, lse_d = bd.sparse_attention(dq, dK, dV, didx, scale, kv_len=dkvl, with_lse=True)
    else:
        lse_d = torch.from_numpy(lse.astype(np.float32)).to(DEV)
    loss, dsc = bd.indexer_kl(dq, dK, didx, lse_d, torch.from_numpy(scores).to(DEV), scale,
                              kv_len=dkvl)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), dsc.cpu().numpy()


def test_kl_sparse_lse_ragged_d128():
    say("[ix_indexer_kl] B=2 T=24 S=700 H_q=16 d=128 k=100, forward lse")
    q, K, V, kvl, idx, sc = _random_case(2, 24, 700, 16, 1, 128, 100, 91, kv_lens=[700, 333],
                                         empty_rows={(1, 5)})
    scale = 128 ** -0.5
    loss, dsc = _gpu_kl(q, K, V, kvl, idx, sc, scale)
    assert loss[1, 5] == 0 and np.all(dsc[1, 5] == 0)
    _check(loss, dsc, idx, sc, q, K, kvl, scale)


def test_kl_sharp_logits_gqa_d64():
    say("[ix_indexer_kl] B=1 T=17 S=2100 H_q=16 H_kv=2 d=64 k=2048 sharp")
    q, K, V, kvl, idx, sc = _random_case(1, 17, 2100, 16, 2, 64, 2048, 92, sharp=6.0)
    scale = 64 ** -0.5
    loss, dsc = _gpu_kl(q, K, V, kvl, idx, sc, scale)
    _check(loss, dsc, idx, sc, q, K, kvl, scale)


def test_kl_dense_lse_and_k_not_multiple_of_4():
    say("[ix_indexer_kl] B=2 T=9 S=300 H_q=8 d=128 k=37, dense lse from the oracle")
    q, K, V, kvl, idx, sc = _random_case(2, 9, 300, 8, 1, 128, 37, 93, kv_lens=[300, 251])
    scale = 128 ** -0.5
    qf = O.decode_bf16(_bits(q))
    Kf = O.decode_bf16(_bits(K))
    lse = np.zeros((2, 9, 8))
    for b in range(2):
        for t in range(9):
            for h in range(8):
                lg = scale * (Kf[b, :kvl[b], 0, :] @ qf[b, t, h])
                lse[b, t, h] = lg.max() + np.log(np.exp(lg - lg.max()).sum())
    loss, dsc = _gpu_kl(q, K, V, kvl, idx, sc, scale, lse=lse)
    _check(loss, dsc, idx, sc, q, K, kvl, scale, lse=lse.astype(np.float32).astype(np.float64))


def test_kl_on_the_indexer_selection():
    """The training chain ix_topk -> sparse_attn_fwd (lse) -> ix_indexer_kl against the
    oracle's own chain.  Indexer codes in {0, +-0.5, +-1} and head weights that are multiples
    of 1/64 make every score exact in fp32, so both sides keep the same keys (ties to the
    lower index) with the same kept scores."""
    B, T, S, H_I, d_I, k, pos0 = 1, 64, 1500, 16, 128, 256, 1436
    say(f"[ix_indexer_kl] ix_topk -> sparse_attn_fwd -> ix_indexer_kl, T={T} S={S} k={k}")
    g = torch.Generator(device="cpu").manual_seed(94)
    vals = torch.tensor([0.0, 0.5, -0.5, 1.0, -1.0])
    qI = synth.encode_e4m3(vals[torch.randint(5, (B, T, H_I, d_I), generator=g)])
    kI = synth.encode_e4m3(vals[torch.randint(5, (B, S, d_I), generator=g)])
    w = torch.randint(-16, 17, (B, T, H_I), generator=g).float() / 64.0
    p0 = torch.tensor([pos0], dtype=torch.int32)
    kvl = torch.tensor([S], dtype=torch.int32)
    q = torch.randn(1, T, 16, 128, generator=g).to(torch.bfloat16)
    K = (torch.randn(1, S, 1, 128, generator=g) * 128 ** -0.5).to(torch.bfloat16)
    V = torch.randn(1, S, 1, 128, generator=g).to(torch.bfloat16)
    scale, temp = 128 ** -0.5, 0.25
    dv = [x.to(DEV) for x in (qI, kI, w, p0, kvl, q, K, V)]
    idx, sel = bd.topk(*dv[:5], k, with_scores=True)
    _, lse = bd.sparse_attention(dv[5], dv[6], dv[7], idx, scale, kv_len=dv[4], with_lse=True)
    loss, dsc = bd.indexer_kl(dv[5], dv[6], idx, lse, (sel * temp).contiguous(), scale,
                              kv_len=dv[4])
    torch.cuda.synchronize()
    rows = list(range(T))
    ref_idx, ref_sc = O.topk_rows(qI.numpy(), kI.numpy(), w.numpy().astype(np.float64),
                                  p0.numpy(), kvl.numpy(), 0, rows, k, return_scores=True)
    assert np.array_equal(idx[0].cpu().numpy(), ref_idx), "selection differs"
    kept = np.full((T, k), -np.inf)
    for t in rows:
        v = ref_idx[t] >= 0
        kept[t, v] = ref_sc[t][ref_idx[t][v]]
    got_sel = sel[0].cpu().numpy().astype(np.float64)
    assert np.array_equal(got_sel, kept), "kept scores differ"
    qb, Kb = _bits(q), _bits(K)
    ref_l, ref_d = O.indexer_kl_rows(qb, Kb, ref_idx, kept * temp, 0, rows, scale, S)
    qf, Kf = O.decode_bf16(qb)[0], O.decode_bf16(Kb)[0]
    got_l, got_d = loss[0].cpu().numpy(), dsc[0].cpu().numpy()
    for t in rows:
        eps, bound = kl_tolerance(qf[t], Kf, ref_idx[t], kept[t] * temp, ref_d[t], scale)
        assert abs(got_l[t] - ref_l[t]) <= eps + 1e-5 * abs(ref_l[t]), f"loss t={t}"
        assert np.all(np.abs(got_d[t] - ref_d[t]) <= bound), f"dscores t={t}"
