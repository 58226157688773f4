"""GPU parity over a fixed, seeded set of random small shapes inside the supported range:
indexer head dim 64/128, indexer heads any multiple of 4, GQA ratios 1..16, attention head
dim 64/128, ragged kv_len (including 0), q_pos0 before the start and late in the cache, k
below and above the visible count, batches large enough for key splits.  Every query row's
selection is checked against the oracle (tie band), and every row where the GPU kept the
oracle's own set has its attention output checked against the oracle on that selection;
grouped shapes go through indexshare_group_fwd.  The same shapes also run IndexPool (pool 4,
k/4 blocks) and the training side (the KL objective, the attention gradients and the indexer
gradients, run on the oracle's selection and the oracle's kept scores), each against the
oracle."""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from indexed_sparse_attention_ix_amd.workloads import Workload
from oracle import ix_oracle as O
from parity_util import (abs_codes, bf16_to_f64, check_attention, check_index_row,
                         check_indexer_bwd, kl_tolerance, oracle_selection, say, to_host_attn,
                         to_host_indexer)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _configs(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.choice([1, 2, 3, 5, 24]))
        T = int(rng.integers(1, 6 if B == 24 else 40))
        S = int(rng.integers(5, 2500))
        d_I = int(rng.choice([64, 128]))
        H_I = 4 * int(rng.integers(1, 17))
        k = int(rng.integers(1, 400))
        H_kv = int(rng.choice([1, 2]))
        grp = int(rng.choice([1, 4, 8, 16]))
        d = int(rng.choice([64, 128]))
        layers = int(rng.choice([1, 3]))
        pos0s = tuple(int(rng.integers(-3, S)) for _ in range(B))
        kv_lens = tuple(int(rng.integers(0, S + 1)) if rng.random() < 0.7 else S for _ in range(B))
        std = float(rng.choice([1.0, d ** -0.5]))
        out.append(Workload(name=f"rand{i}", B=B, T=T, S=S, pos0=0, H_I=H_I, d_I=d_I, k=k,
                            H_q=H_kv * grp, H_kv=H_kv, d=d, layers=layers, seed=300 + i,
                            qkv_std=std, planted=int(rng.choice([0, 4])), kv_lens=kv_lens,
                            pos0s=pos0s))
    return out


@pytest.mark.parametrize("wl", _configs(), ids=lambda w: w.name)
def test_random_shape(wl):
    say(f"[random shape] {wl.name}: B={wl.B} T={wl.T} S={wl.S} H_I={wl.H_I} d_I={wl.d_I} k={wl.k} "
        f"H_q={wl.H_q} H_kv={wl.H_kv} d={wl.d} layers={wl.layers} pos0={wl.pos0s} kv_len={wl.kv_lens}")
    ind = synth.indexer_inputs(wl, device=DEV)
    layers = [synth.attention_inputs(wl, layer=l, device=DEV) for l in range(wl.layers)]
    args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    if wl.layers > 1:
        idx, outs, lses = bd.indexshare_group(*args, wl.k, [dict(q=L["q"], K=L["K"], V=L["V"])
                                                            for L in layers], wl.sm_scale,
                                              with_lse=True)
    else:
        idx = bd.topk(*args, wl.k)
        o, l0 = bd.sparse_attention(layers[0]["q"], layers[0]["K"], layers[0]["V"], idx,
                                    wl.sm_scale, kv_len=ind["kv_len"], with_lse=True)
        outs, lses = [o], [l0]
    torch.cuda.synchronize()
    h = to_host_indexer(ind)
    idx_np = idx.cpu().numpy()
    ref_idx, same = [], []
    for b in range(wl.B):
        keys = O.decode_e4m3(h["k_I"][b])
        ns = [O.visible_count(h["q_pos0"][b], h["kv_len"][b], t) for t in range(wl.T)]
        scs = [O.score_row(h["q_I"][b, t], keys[:ns[t]], h["w"][b, t], ns[t]) for t in range(wl.T)]
        r, m = oracle_selection(idx_np[b], scs, wl.k, ns, where=f"{wl.name} b={b}")
        ref_idx.append(r)
        same.append(m)
    n_same = int(sum(m.sum() for m in same))
    assert n_same >= 0.9 * wl.B * wl.T, f"{wl.name}: only {n_same} rows kept the oracle's own set"
    for l, L in enumerate(layers):
        hl = to_host_attn(L)
        for b in range(wl.B):
            ref_o, ref_l = O.sparse_attention_rows(hl["q"], hl["K"], hl["V"], ref_idx[b], b,
                                                   list(range(wl.T)), wl.sm_scale)
            m = same[b]
            if not m.any():
                continue
            check_attention(bf16_to_f64(outs[l])[b][m], ref_o[m], lses[l].cpu().numpy()[b][m],
                            ref_l[m], where=f"{wl.name} layer={l} b={b}")


@pytest.mark.parametrize("wl", _configs()[:12], ids=lambda w: w.name)
def test_random_shape_indexpool(wl):
    pool, kb = 4, max(1, wl.k // 4)
    say(f"[random shape IndexPool] {wl.name}: B={wl.B} T={wl.T} S={wl.S} k_blocks={kb}")
    ind = synth.indexer_inputs(wl, device=DEV)
    kp = bd.pool_keys(ind["k_I"], ind["kv_len"], pool)
    idx = bd.topk_pooled(ind["q_I"], kp, ind["w"], ind["q_pos0"], ind["kv_len"], wl.S, pool, kb)
    torch.cuda.synchronize()
    h = to_host_indexer(ind)
    kp_h, got = kp.cpu().numpy(), idx.cpu().numpy()
    for b in range(wl.B):
        ref_kp = O.pool_keys(h["k_I"][b], int(h["kv_len"][b]), pool)
        assert np.array_equal(kp_h[b], ref_kp), f"block keys b={b}"
        pooled = O.decode_e4m3(ref_kp)
        for t in range(wl.T):
            pos0, kvl = int(h["q_pos0"][b]), int(h["kv_len"][b])
            sc, _, _ = O.pooled_topk_row(h["q_I"][b, t], pooled, h["w"][b, t], pos0, kvl, t, pool, kb)
            row = got[b, t]
            blocks = sorted(set((row[row >= 0] // pool).tolist()))
            padded = np.full(kb, -1, dtype=np.int64)
            padded[:len(blocks)] = blocks
            check_index_row(padded, sc, kb, len(sc), where=f"{wl.name} b={b} t={t}")
            n_t = O.visible_count(pos0, kvl, t)
            toks = [pool * j + r for j in blocks for r in range(pool) if pool * j + r < n_t]
            want = np.full(kb * pool, -1, dtype=np.int64)
            want[:len(toks)] = toks
            assert np.array_equal(row, want), f"expansion {wl.name} b={b} t={t}"


@pytest.mark.parametrize("wl", _configs()[:12], ids=lambda w: w.name)
def test_random_shape_training(wl):
    """The training side on the oracle's own selection and kept scores (ix_topk's selection
    is checked against them first): KL loss and score gradient per row within the KL
    tolerance; dq per row and dK, dV per sequence within 2e-2 relative in norm plus a floor
    of 1e-4 sqrt(n) times one term's size (bf16 P and dS in the products); the indexer
    gradients per entry (check_indexer_bwd) with the KL tolerance carried through."""
    say(f"[random shape training] {wl.name}: B={wl.B} T={wl.T} S={wl.S} H_q={wl.H_q} "
        f"H_kv={wl.H_kv} d={wl.d} k={wl.k}")
    ind = synth.indexer_inputs(wl, device=DEV)
    att = synth.attention_inputs(wl, layer=0, device=DEV)
    args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    idx = bd.topk(*args, wl.k)
    torch.cuda.synchronize()
    h = to_host_indexer(ind)
    idx_np = idx.cpu().numpy()
    ref_idx = np.full((wl.B, wl.T, wl.k), -1, dtype=np.int32)
    kept = np.full((wl.B, wl.T, wl.k), -np.inf)
    for b in range(wl.B):
        keys = O.decode_e4m3(h["k_I"][b])
        ns = [O.visible_count(h["q_pos0"][b], h["kv_len"][b], t) for t in range(wl.T)]
        scs = [O.score_row(h["q_I"][b, t], keys[:ns[t]], h["w"][b, t], ns[t]) for t in range(wl.T)]
        r, _ = oracle_selection(idx_np[b], scs, wl.k, ns, where=f"{wl.name} b={b}")
        ref_idx[b] = r
        for t in range(wl.T):
            v = r[t] >= 0
            kept[b, t, v] = scs[t][r[t][v]]
    finite = kept[np.isfinite(kept)]
    temp = 1.0 / max(float(finite.std()), 1e-3) if finite.size > 1 else 1.0
    kept_t = (kept * temp).astype(np.float32)            # the scores both sides use
    ridx = torch.from_numpy(ref_idx).to(DEV)
    out, lse = bd.sparse_attention(att["q"], att["K"], att["V"], ridx, wl.sm_scale,
                                   kv_len=ind["kv_len"], with_lse=True)
    loss, dsc = bd.indexer_kl(att["q"], att["K"], ridx, lse, torch.from_numpy(kept_t).to(DEV),
                              wl.sm_scale, kv_len=ind["kv_len"])
    g = torch.Generator(device="cpu").manual_seed(wl.seed)
    dout = torch.randn(att["q"].shape, generator=g).to(torch.bfloat16).to(DEV)
    dq, dK, dV = bd.sparse_attention_backward(att["q"], att["K"], att["V"], ridx, out, lse, dout,
                                              wl.sm_scale, kv_len=ind["kv_len"])
    ib = bd.indexer_bwd(bd.indexer_args(*args), ridx, dsc, DEV)
    # the atomic-free forms, in passes of 3 query rows
    dq3, dK3, dV3 = bd.sparse_attention_backward(att["q"], att["K"], att["V"], ridx, out, lse, dout,
                                                 wl.sm_scale, kv_len=ind["kv_len"], rows_per_pass=3)
    ib3 = bd.indexer_bwd(bd.indexer_args(*args), ridx, dsc, DEV, rows_per_pass=3)
    torch.cuda.synchronize()
    assert torch.equal(dq3, dq) and torch.equal(ib3[0], ib[0]) and torch.equal(ib3[1], ib[1])
    hl = to_host_attn(att)
    kvl = h["kv_len"]
    sc_np = kept_t.astype(np.float64)
    loss_np, dsc_np = loss.cpu().numpy(), dsc.cpu().numpy()
    dq_np, dK_np, dV_np = dq.cpu().numpy(), dK.cpu().numpy(), dV.cpu().numpy()
    dout_np = dout.float().cpu().numpy().astype(np.float64)
    qf, Kf = O.decode_bf16(hl["q"]), O.decode_bf16(hl["K"])
    term = wl.sm_scale * float(np.abs(Kf).max() * np.abs(dout_np).max() *
                               np.abs(O.decode_bf16(hl["V"])).max())

    def close(g_, r_, what):
        err = np.linalg.norm(g_ - r_)
        assert err <= 2e-2 * np.linalg.norm(r_) + 1e-4 * term * np.sqrt(r_.size), \
            f"{wl.name} {what}: {err:.3e} vs {np.linalg.norm(r_):.3e}"

    ref_ds = np.zeros((wl.B, wl.T, wl.k))
    carried = []
    for b in range(wl.B):
        rl, rd = O.indexer_kl_rows(hl["q"], hl["K"], ref_idx[b], sc_np[b], b, list(range(wl.T)),
                                   wl.sm_scale, int(kvl[b]))
        ref_ds[b] = rd
        rq, rK, rV = O.sparse_attention_backward_rows(hl["q"], hl["K"], hl["V"], ref_idx[b],
                                                      dout_np[b], b, list(range(wl.T)), wl.sm_scale)
        eps_ds = np.zeros((wl.T, wl.k))
        for t in range(wl.T):
            eps, bound = kl_tolerance(qf[b, t], Kf[b], ref_idx[b, t], sc_np[b, t], rd[t], wl.sm_scale)
            eps_ds[t] = bound
            assert abs(loss_np[b, t] - rl[t]) <= eps + 1e-5 * abs(rl[t]), f"{wl.name} KL b={b} t={t}"
            assert np.all(np.abs(dsc_np[b, t] - rd[t]) <= bound), f"{wl.name} dscores b={b} t={t}"
            if (ref_idx[b, t] < 0).all():
                assert np.all(dq_np[b, t] == 0)
            else:
                close(dq_np[b, t], rq[t], f"dq b={b} t={t}")
        close(dK_np[b], rK, f"dK b={b}")
        close(dV_np[b], rV, f"dV b={b}")
        close(dK3[b].cpu().numpy(), rK, f"dK (atomic-free) b={b}")
        close(dV3[b].cpu().numpy(), rV, f"dV (atomic-free) b={b}")
        carried.append(O.indexer_backward_rows(abs_codes(h["q_I"]), abs_codes(h["k_I"]),
                                               np.abs(h["w"]), ref_idx[b], eps_ds, b,
                                               list(range(wl.T)), int(kvl[b])))
    check_indexer_bwd(tuple(x.cpu().numpy() for x in ib), h["q_I"], h["k_I"], h["w"], ref_idx,
                      ref_ds, kvl, extra=carried, where=wl.name)
    check_indexer_bwd(tuple(x.cpu().numpy() for x in ib3), h["q_I"], h["k_I"], h["w"], ref_idx,
                      ref_ds, kvl, extra=carried, where=wl.name + " (atomic-free)", bf16_rows=True)
