"""GPU parity of the training side at the 32K prefill's full size (T = S = 32,768, k = 2048,
16 query heads over one KV head), in the configuration the benchmark times: ix_topk with
the kept scores, sparse_attn_fwd with lse, then ix_indexer_kl and sparse_attn_bwd.

Sampled queries are checked one by one against the oracle on the GPU's own index tensor
(KL loss and score gradient; dq).  dK and dV sum over every query that kept a row, which the
oracle cannot sample, so they are checked through two identities of the softmax chain rule
that hold at any size: for each query and head the row gradients dl_j = p_j (dp_j - D) sum
to zero, so sum_j dK_j = 0; and sum_j p_j = 1, so sum_j dV_j = the sum of dout over the
(query, head) pairs with a non-empty selection.  Tolerances as the small-size tests: per
query 2e-2 relative in norm for dq (bf16 P and dS in the products), KL as
test_gpu_indexer_kl; the identities within 1e-2 of the gradients' own size.
"""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from indexed_sparse_attention_ix_amd.workloads import WORKLOADS
from oracle import ix_oracle as O
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


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
    # kept scores are large (hundreds); a fixed temperature keeps the prediction soft
    sel_t = (sel * 0.01).contiguous()
    say("  ix_indexer_kl")
    loss, dsc = bd.indexer_kl(att["q"], att["K"], idx, lse, sel_t, wl.sm_scale,
                              kv_len=ind["kv_len"])
    g = torch.Generator(device="cpu").manual_seed(7)
    dout = torch.randn(att["q"].shape, generator=g).to(torch.bfloat16).to(DEV)
    say("  sparse_attn_bwd")
    dq, dK, dV = bd.sparse_attention_backward(att["q"], att["K"], att["V"], idx, out, lse, dout,
                                              wl.sm_scale, kv_len=ind["kv_len"])
    torch.cuda.synchronize()

    rng = np.random.default_rng(321)
    rows = sorted(set([0, 1, wl.k - 1, wl.k, wl.T - 1]) |
                  set(rng.choice(wl.T, size=27, replace=False).tolist()))
    say(f"  oracle on {len(rows)} rows")
    q_bits = synth.bf16_bits(att["q"][0, rows])[None]
    K_bits = synth.bf16_bits(att["K"][0])[None]
    V_bits = synth.bf16_bits(att["V"][0])[None]
    idx_r = idx[0, rows].cpu().numpy()
    sc_r = sel_t[0, rows].cpu().numpy().astype(np.float64)
    kvl = int(ind["kv_len"][0].item())

    # KL: loss and score gradient per sampled query
    ref_l, ref_d = O.indexer_kl_rows(q_bits, K_bits, idx_r, sc_r, 0, list(range(len(rows))),
                                     wl.sm_scale, kvl)
    got_l = loss[0, rows].cpu().numpy()
    got_d = dsc[0, rows].cpu().numpy()
    qf = O.decode_bf16(q_bits)[0]
    Kf = O.decode_bf16(K_bits)[0]
    for i, t in enumerate(rows):
        v = idx_r[i][(idx_r[i] >= 0) & (idx_r[i] < kvl)]
        L = float(np.abs(wl.sm_scale * (Kf[v, 0, :] @ qf[i].T)).max())
        eps = 2e-5 * (1 + L)
        assert abs(got_l[i] - ref_l[i]) <= eps + 1e-5 * abs(ref_l[i]), f"KL loss t={t}"
        valid = (idx_r[i] >= 0) & (idx_r[i] < kvl)
        e = np.exp(sc_r[i][valid] - sc_r[i][valid].max())
        pred = np.zeros(wl.k)
        pred[valid] = e / e.sum()
        bound = eps * np.maximum(pred, np.abs(pred - ref_d[i])) + 1e-7
        assert np.all(np.abs(got_d[i] - ref_d[i]) <= bound), f"KL dscores t={t}"

    # dq per sampled query
    dout_r = dout[0, rows].float().cpu().numpy().astype(np.float64)
    ref_dq, _, _ = O.sparse_attention_backward_rows(q_bits, K_bits, V_bits, idx_r, dout_r, 0,
                                                    list(range(len(rows))), wl.sm_scale)
    got_dq = dq[0, rows].cpu().numpy()
    term = wl.sm_scale * float(att["K"].float().abs().max() * dout.float().abs().max() *
                               att["V"].float().abs().max())
    for i, t in enumerate(rows):
        err = np.linalg.norm(got_dq[i] - ref_dq[i])
        assert err <= 2e-2 * np.linalg.norm(ref_dq[i]) + 1e-4 * term * np.sqrt(ref_dq[i].size), \
            f"dq t={t}: {err:.3e} vs {np.linalg.norm(ref_dq[i]):.3e}"

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
    say(f"  ok; |sum dV - want| / |want| = {float((got_dv - want_dv).norm() / want_dv.norm()):.2e}, "
        f"|sum dK| / |dK| = {float(sum_dk.norm() / dK64.norm()):.2e}")
