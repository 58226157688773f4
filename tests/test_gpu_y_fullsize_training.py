"""GPU parity of the training side at the 32K prefill's full size (T = S = 32,768, k = 2048,
16 query heads over one KV head, 64 indexer heads), in the configuration the benchmark
times: ix_topk with the kept scores, sparse_attn_fwd with lse, then ix_indexer_kl,
sparse_attn_bwd and ix_indexer_bwd.

Sampled queries are checked one by one against the oracle's own chain: its selection (the
GPU's is checked against the oracle's scores; rows where the GPU kept another, equally
valid set are left out of the checks downstream), its kept scores (which the GPU's KL is
given for those rows, so that both sides start from the same values), the KL loss and score
gradient, the attention's dq, and the indexer's dq_I and dw with the KL tolerance carried
through.  dK, dV and dk_I sum over every query that kept a row, which the oracle cannot
sample.  So the test also builds a probe selection: the sampled rows keep the oracle's
selection, and a set of probe keys taken from it is removed from every other row, so the
probe keys' gradients are sums over sampled rows only.  The full-size kernels then run on
that selection, and every entry of dq (sampled rows) and of dK, dV and dk_I (probe keys) is
checked against the oracle, in both backward forms.  Identities that hold at any size check
all keys besides: for each query and head the row gradients dl_j = p_j (dp_j - D) sum to
zero, so sum_j dK_j = 0; sum_j p_j = 1, so sum_j dV_j = the sum of dout over the (query,
head) pairs with a non-empty selection; and the score is linear in w and positively
homogeneous of degree 1 in q_I and in k_I, so <dk_I, k_I> = <dq_I, q_I> = <dw, w>.
Tolerances: the attention gradients per entry as test_gpu_attention_bwd, KL as
test_gpu_indexer_kl, the indexer gradients per entry as test_gpu_indexer_bwd; the attention
identities within 1e-2 of the gradients' own size, the indexer identity within 1e-3 of the
sum of |terms|.
"""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from indexed_sparse_attention_ix_amd.workloads import WORKLOADS
from oracle import ix_oracle as O
from parity_util import (FP32_U, abs_codes, attn_bwd_bounds, indexer_bwd_coefficients,
                         check_attn_bwd_entries, kl_tolerance, logit_magnitude, oracle_selection,
                         say)

pytestmark = pytest.mark.gpu
DEV = "cuda"
TEMP = 0.01   # kept scores are large (hundreds); a fixed temperature keeps the prediction soft


def test_prefill_32k_kl_and_backward_full_size():
    wl = WORKLOADS["prefill_32k"]
    say(f"[full size training] prefill_32k: T={wl.T} S={wl.S} k={wl.k} H_q={wl.H_q} d={wl.d}")
    ind = synth.indexer_inputs(wl, device=DEV)
    att = synth.attention_inputs(wl, layer=0, device=DEV)
    args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    say("  ix_topk with kept scores, sparse_attn_fwd with lse")
    idx, sel = bd.topk(*args, wl.k, with_scores=True)
    out, lse = bd.sparse_attention(att["q"], att["K"], att["V"], idx, wl.sm_scale,
                                   kv_len=ind["kv_len"], with_lse=True)
    torch.cuda.synchronize()

    rng = np.random.default_rng(321)
    rows = sorted(set([0, 1, wl.k - 2, wl.k - 1, wl.k, wl.T - 1]) |
                  set(rng.choice(wl.T, size=26, replace=False).tolist()))
    say(f"  oracle selection on {len(rows)} rows")
    qI_h = ind["q_I"].cpu().numpy()
    kI_h = ind["k_I"].cpu().numpy()
    w_h = ind["w"].cpu().numpy()
    pos0 = int(ind["q_pos0"][0].item())
    kvl = int(ind["kv_len"][0].item())
    keys = O.decode_e4m3(kI_h[0])
    ns = [O.visible_count(pos0, kvl, t) for t in rows]
    scs = [O.score_row(qI_h[0, t], keys[:n], w_h[0, t], n) for t, n in zip(rows, ns)]
    ref_idx, same = oracle_selection(idx[0, rows].cpu().numpy(), scs, wl.k, ns, where="32K")
    assert same.mean() >= 0.9, f"{int((~same).sum())} of {len(rows)} rows kept another tied set"
    kept = np.full((len(rows), wl.k), -np.inf)
    for i in range(len(rows)):
        v = ref_idx[i] >= 0
        kept[i, v] = scs[i][ref_idx[i][v]]
    kept_t = (kept * TEMP).astype(np.float32)
    # the GPU's KL gets the oracle's kept scores on the sampled rows where the sets agree
    sel_t = (sel * TEMP).contiguous()
    rows_same = [t for t, m in zip(rows, same) if m]
    sel_t[0, rows_same] = torch.from_numpy(kept_t[same]).to(DEV)

    say("  ix_indexer_kl, sparse_attn_bwd, ix_indexer_bwd")
    loss, dsc = bd.indexer_kl(att["q"], att["K"], idx, lse, sel_t, wl.sm_scale,
                              kv_len=ind["kv_len"])
    g = torch.Generator(device="cpu").manual_seed(7)
    dout = torch.randn(att["q"].shape, generator=g).to(torch.bfloat16).to(DEV)
    dq, dK, dV = bd.sparse_attention_backward(att["q"], att["K"], att["V"], idx, out, lse, dout,
                                              wl.sm_scale, kv_len=ind["kv_len"])
    dq_I, dw, dk_I = bd.indexer_bwd(bd.indexer_args(*args), idx, dsc, DEV)
    torch.cuda.synchronize()

    say(f"  oracle chain on {int(same.sum())} rows")
    sub = [i for i in range(len(rows)) if same[i]]
    q_bits = synth.bf16_bits(att["q"][0, rows])[None]
    K_bits = synth.bf16_bits(att["K"][0])[None]
    V_bits = synth.bf16_bits(att["V"][0])[None]
    ref_l, ref_d = O.indexer_kl_rows(q_bits, K_bits, ref_idx, kept_t.astype(np.float64), 0,
                                     list(range(len(rows))), wl.sm_scale, kvl)
    got_l = loss[0, rows].cpu().numpy()
    got_d = dsc[0, rows].cpu().numpy()
    qf = O.decode_bf16(q_bits)[0]
    Kf = O.decode_bf16(K_bits)[0]
    eps_ds = np.zeros((len(rows), wl.k))
    for i in sub:
        eps, bound = kl_tolerance(qf[i], Kf, ref_idx[i], kept_t[i], ref_d[i], wl.sm_scale)
        eps_ds[i] = bound
        assert abs(got_l[i] - ref_l[i]) <= eps + 1e-5 * abs(ref_l[i]), f"KL loss t={rows[i]}"
        assert np.all(np.abs(got_d[i] - ref_d[i]) <= bound), f"KL dscores t={rows[i]}"

    # attention dq per sampled query
    dout_r = dout[0, rows].float().cpu().numpy().astype(np.float64)
    ref_dq, _, _ = O.sparse_attention_backward_rows(q_bits, K_bits, V_bits, ref_idx, dout_r, 0,
                                                    list(range(len(rows))), wl.sm_scale)
    mags = O.sparse_attention_backward_magnitudes(q_bits, K_bits, V_bits, ref_idx, dout_r, 0,
                                                  list(range(len(rows))), wl.sm_scale)
    got_dq = dq[0, rows].cpu().numpy()
    lmag = logit_magnitude(qf, Kf, wl.sm_scale)
    bound_dq = attn_bwd_bounds(mags, wl.k, wl.T, wl.H_q, wl.d, lmag, False)[0]
    check_attn_bwd_entries(got_dq[sub], ref_dq[sub], bound_dq[sub], "dq (sampled rows)",
                           power=0.5)

    # indexer dq_I and dw per sampled query (dk_I through the identity below)
    qI_r = qI_h[0, rows][None]
    w_r = w_h[0, rows][None]
    r_dq, r_dw, _ = O.indexer_backward_rows(qI_r, kI_h, w_r, ref_idx, ref_d, 0,
                                            list(range(len(rows))), kvl)
    m_dq, m_dw, _ = O.indexer_backward_rows(abs_codes(qI_r), abs_codes(kI_h), np.abs(w_r),
                                            ref_idx, np.abs(ref_d), 0, list(range(len(rows))), kvl)
    c_dq, c_dw, _ = O.indexer_backward_rows(abs_codes(qI_r), abs_codes(kI_h), np.abs(w_r),
                                            ref_idx, eps_ds, 0, list(range(len(rows))), kvl)
    coef_I = indexer_bwd_coefficients(wl.k, wl.T)
    g_dq = dq_I[0, rows].cpu().numpy().astype(np.float64)
    g_dw = dw[0, rows].cpu().numpy().astype(np.float64)
    for i in sub:
        b_dq = coef_I[0] * m_dq[i] + c_dq[i]
        b_dw = coef_I[1] * m_dw[i] + c_dw[i]
        assert np.all(np.abs(g_dq[i] - r_dq[i]) <= b_dq), f"dq_I t={rows[i]}"
        assert np.all(np.abs(g_dw[i] - r_dw[i]) <= b_dw), f"dw t={rows[i]}"

    # dK and dV through the identities
    dK64 = dK[0, :, 0].double()
    dV64 = dV[0, :, 0].double()
    has_rows = ((idx[0] >= 0) & (idx[0] < kvl)).any(dim=1)            # [T]
    want_dv = (dout[0].double() * has_rows[:, None, None]).sum(dim=(0, 1))  # [d]
    got_dv = dV64.sum(dim=0)
    assert float((got_dv - want_dv).norm()) <= 1e-2 * float(want_dv.norm()) + 1e-3, "sum of dV"
    sum_dk = dK64.sum(dim=0)
    assert float(sum_dk.norm()) <= 1e-2 * float(dK64.norm()), \
        f"sum of dK {float(sum_dk.norm()):.3e} vs |dK| {float(dK64.norm()):.3e}"

    # the indexer gradients through <dk_I, k_I> = <dq_I, q_I> = <dw, w>
    qv = synth.decode_e4m3_torch(ind["q_I"]).double()
    kv = synth.decode_e4m3_torch(ind["k_I"]).double()
    t_q = dq_I.double() * qv
    t_k = dk_I.double() * kv
    t_w = dw.double() * ind["w"].double()
    e_q, e_k, e_w = float(t_q.sum()), float(t_k.sum()), float(t_w.sum())
    scale_id = float(t_q.abs().sum() + t_k.abs().sum() + t_w.abs().sum())
    assert abs(e_q - e_w) <= 1e-3 * scale_id and abs(e_k - e_w) <= 1e-3 * scale_id, \
        f"indexer identity: <dq,q> {e_q:.6e} <dk,k> {e_k:.6e} <dw,w> {e_w:.6e}"
    # the atomic-free forms (inverted selection, per-pair bf16 rows, key-major sums), in four
    # passes: dq, dq_I and dw are the same computation; the key gradients agree to the bf16
    # rounding of each pair's rows
    say("  atomic-free sparse_attn_bwd and ix_indexer_bwd, 8192 rows per pass")
    dq2, dK2, dV2 = bd.sparse_attention_backward(att["q"], att["K"], att["V"], idx, out, lse, dout,
                                                 wl.sm_scale, kv_len=ind["kv_len"],
                                                 rows_per_pass=8192)
    dq_I2, dw2, dk_I2 = bd.indexer_bwd(bd.indexer_args(*args), idx, dsc, DEV, rows_per_pass=8192)
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq) and torch.equal(dq_I2, dq_I) and torch.equal(dw2, dw)
    for x, y, nm in ((dK, dK2, "dK"), (dV, dV2, "dV"), (dk_I, dk_I2, "dk_I")):
        err = float((x.double() - y.double()).norm())
        assert err <= 4e-3 * float(x.double().norm()), f"{nm}: {err:.3e}"
    say(f"  ok; |sum dV - want| / |want| = {float((got_dv - want_dv).norm() / want_dv.norm()):.2e}, "
        f"|sum dK| / |dK| = {float(sum_dk.norm() / dK64.norm()):.2e}, indexer identity "
        f"{max(abs(e_q - e_w), abs(e_k - e_w)) / scale_id:.2e} of the sum of |terms|")
    del dq2, dK2, dV2, dq_I2, dw2, dk_I2, dK, dV, dk_I

    # ------------------------------------------------------------------ probe keys
    # The sampled rows keep the oracle's selection; probe keys drawn from it (two per sampled
    # row, plus keys 0 and 1, which the first rows keep) are removed from every other row.
    # A probe key's dK, dV and dk_I are then sums over sampled rows, which the oracle forms
    # exactly.  The selection changes, so the forward runs again on it; the KL's score
    # gradient on the sampled rows is the oracle's (an oracle -> GPU input, rounded to fp32
    # for both sides).
    prng = np.random.default_rng(654)
    probes = {0, 1}
    for i in range(len(rows)):
        v = ref_idx[i][ref_idx[i] >= 0]
        probes |= set(prng.choice(v, size=min(2, len(v)), replace=False).tolist())
    probes = np.array(sorted(probes), dtype=np.int64)
    say(f"  probe selection: {len(probes)} probe keys kept only by the {len(rows)} sampled rows")
    idx2 = idx.clone()
    idx2[0, rows] = torch.from_numpy(ref_idx.astype(np.int32)).to(DEV)
    sampled = torch.zeros(wl.T, dtype=torch.bool, device=DEV)
    sampled[rows] = True
    probes_t = torch.from_numpy(probes).to(DEV)
    drop = torch.isin(idx2[0], probes_t) & ~sampled[:, None]
    idx2[0][drop] = -1
    del drop
    out2, lse2 = bd.sparse_attention(att["q"], att["K"], att["V"], idx2, wl.sm_scale,
                                     kv_len=ind["kv_len"], with_lse=True)
    dsc2 = dsc.clone()
    ref_d32 = ref_d.astype(np.float32)
    dsc2[0, rows] = torch.from_numpy(ref_d32).to(DEV)
    forms = {}
    for form, rpp in (("atomics", None), ("atomic-free", 8192)):
        g3 = bd.sparse_attention_backward(att["q"], att["K"], att["V"], idx2, out2, lse2, dout,
                                          wl.sm_scale, kv_len=ind["kv_len"], rows_per_pass=rpp)
        i3 = bd.indexer_bwd(bd.indexer_args(*args), idx2, dsc2, DEV, rows_per_pass=rpp)
        torch.cuda.synchronize()
        forms[form] = (g3[0][0, rows].cpu().numpy(),
                       g3[1][0, probes_t, 0].cpu().numpy(), g3[2][0, probes_t, 0].cpu().numpy(),
                       i3[2][0, probes_t].cpu().numpy().astype(np.float64))
        del g3, i3
    # every probe key is kept by sampled rows only
    kept_by = torch.isin(idx2[0][~sampled], probes_t).any()
    assert not bool(kept_by), "a probe key is still kept by a row outside the sample"
    all_rows = list(range(len(rows)))
    r_dq, r_dK, r_dV = O.sparse_attention_backward_rows(q_bits, K_bits, V_bits, ref_idx, dout_r, 0,
                                                        all_rows, wl.sm_scale)
    mags = O.sparse_attention_backward_magnitudes(q_bits, K_bits, V_bits, ref_idx, dout_r, 0,
                                                  all_rows, wl.sm_scale)
    rI = O.indexer_backward_rows(qI_r, kI_h, w_r, ref_idx, ref_d32.astype(np.float64), 0,
                                 all_rows, kvl)[2]
    mI = O.indexer_backward_rows(abs_codes(qI_r), abs_codes(kI_h), np.abs(w_r), ref_idx,
                                 np.abs(ref_d32.astype(np.float64)), 0, all_rows, kvl)[2]
    n_probe_rows = len(rows)
    for form, (g_dq, g_dK, g_dV, g_dkI) in forms.items():
        pair = form == "atomic-free"
        b_dq, b_dK, b_dV = attn_bwd_bounds(mags, wl.k, n_probe_rows, wl.H_q, wl.d, lmag, pair)
        w1 = check_attn_bwd_entries(g_dq, r_dq, b_dq, f"{form} dq (sampled rows)", power=0.5)
        w2 = check_attn_bwd_entries(g_dK, r_dK[probes, 0], b_dK[probes, 0],
                                    f"{form} dK (probe keys)", power=0.5)
        w3 = check_attn_bwd_entries(g_dV, r_dV[probes, 0], b_dV[probes, 0],
                                    f"{form} dV (probe keys)", power=0.5)
        c_kI = indexer_bwd_coefficients(wl.k, n_probe_rows, pair)[2]
        w4 = check_attn_bwd_entries(g_dkI, rI[probes], c_kI * mI[probes],
                                    f"{form} dk_I (probe keys)", power=0.5)
        say(f"  {form}: worst err / bound: dq {w1:.2e}, dK {w2:.2e}, dV {w3:.2e}, dk_I {w4:.2e}")
