"""GPU parity: IndexShare group driver (indexshare_group_fwd)."""
import math

import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from indexed_sparse_attention_ix_amd.workloads import Workload
from oracle import ix_oracle as O
from parity_util import (bf16_to_f64, check_attention, oracle_selection, say, to_host_attn,
                         to_host_indexer)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _group_case(**kw):
    base = dict(name="group", B=2, T=150, S=3000, pos0=0, pos0s=(2850, 1000), kv_lens=(3000, 2500),
                H_I=64, d_I=128, k=256, H_q=16, H_kv=1, d=128, layers=4, seed=41,
                qkv_std=1.0 / math.sqrt(128), planted=8)
    base.update(kw)
    return Workload(**base)


def _close_to_standalone(o, lse, o2, l2, k, where):
    """A layer's output from a launch that splits the selection differently from the
    standalone call's: each split rounds P to bf16 against its own running maximum, so the
    two differ by bf16 roundings of the terms (random in sign, so per (row, head) in norm
    within 2^-5 of the output), and lse by fp32 sums of the k weights in another order
    ((k + 64) 2^-23)."""
    a, b = o.double(), o2.double()
    num, den = (a - b).norm(dim=-1), b.norm(dim=-1)
    assert bool((num <= 2.0 ** -5 * den + 1e-7).all()), \
        f"{where}: worst relative difference {float((num / den.clamp(min=1e-30)).max()):.3e}"
    fin = torch.isfinite(l2)
    assert torch.equal(fin, torch.isfinite(lse))
    assert bool(((lse - l2).abs()[fin] <= (k + 64) * 2.0 ** -23 * (1 + l2.abs()[fin])).all()), \
        f"{where} lse"


def _same_as_group_attention(layers, idx, kv_len, sm_scale, outs, lses):
    """The group's outputs are sparse_attn_group_fwd's on the same selection, bit for bit,
    and each layer's standalone sparse_attn_fwd's up to a different split of the selection."""
    go, gl = bd.group_attention([dict(q=L["q"], K=L["K"], V=L["V"]) for L in layers], idx,
                                sm_scale, kv_len=kv_len, with_lse=True)
    k = idx.shape[-1]
    for l, L in enumerate(layers):
        assert torch.equal(outs[l], go[l]) and torch.equal(lses[l], gl[l]), f"layer {l}"
        o2, l2 = bd.sparse_attention(L["q"], L["K"], L["V"], idx, sm_scale, kv_len=kv_len,
                                     with_lse=True)
        _close_to_standalone(outs[l], lses[l], o2, l2, k, f"layer {l}")


def test_group_attention_entry_point_against_standalone_and_oracle():
    """sparse_attn_group_fwd on a caller's selection, against standalone calls and the oracle:
    a ragged prefill of 1200 query rows (one launch per layer with the standalone call's
    split: bit for bit), and two small batches whose layers share one launch of the light
    kernel (a standalone call runs the other kernel: within the split-rounding bound): 300
    ragged query rows, and a decode batch."""
    for case in (dict(B=2, T=600, S=3000, pos0s=(2400, 1000), kv_lens=(3000, 2500), k=256,
                      layers=3, seed=45),
                 dict(B=2, T=150, S=3000, pos0s=(2850, 1000), kv_lens=(3000, 2500), k=256,
                      layers=3, seed=47),
                 dict(B=8, T=1, S=9000, pos0=8999, pos0s=None, kv_lens=None, k=2048, layers=3,
                      seed=46, planted=16)):
        wl = _group_case(**case)
        say(f"[sparse_attn_group_fwd] B={wl.B} T={wl.T} S={wl.S} k={wl.k} layers={wl.layers}")
        ind = synth.indexer_inputs(wl, device=DEV)
        layers = [synth.attention_inputs(wl, layer=l, device=DEV) for l in range(wl.layers)]
        args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
        idx = bd.topk(*args, wl.k)
        outs, lses = bd.group_attention([dict(q=L["q"], K=L["K"], V=L["V"]) for L in layers],
                                        idx, wl.sm_scale, kv_len=ind["kv_len"], with_lse=True)
        for l, L in enumerate(layers):
            o2, l2 = bd.sparse_attention(L["q"], L["K"], L["V"], idx, wl.sm_scale,
                                         kv_len=ind["kv_len"], with_lse=True)
            if wl.B * wl.T >= 1024:
                assert torch.equal(outs[l], o2) and torch.equal(lses[l], l2), f"layer {l}"
            else:
                _close_to_standalone(outs[l], lses[l], o2, l2, wl.k, f"layer {l}")
        torch.cuda.synchronize()
        h = to_host_indexer(ind)
        idx_np = idx.cpu().numpy()
        for b in range(wl.B):
            keys = O.decode_e4m3(h["k_I"][b])
            rows = list(range(0, wl.T, 7)) + [wl.T - 1]
            ns = [O.visible_count(h["q_pos0"][b], h["kv_len"][b], t) for t in rows]
            scs = [O.score_row(h["q_I"][b, t], keys[:n], h["w"][b, t], n) for t, n in zip(rows, ns)]
            ref_idx, same = oracle_selection(idx_np[b, rows], scs, wl.k, ns, where=f"b={b}")
            for l in range(wl.layers):
                hl = to_host_attn(layers[l])
                ref_o, ref_l = O.sparse_attention_rows(hl["q"], hl["K"], hl["V"], ref_idx, b, rows,
                                                       wl.sm_scale)
                check_attention(bf16_to_f64(outs[l])[b][rows][same], ref_o[same],
                                lses[l].cpu().numpy()[b][rows][same], ref_l[same],
                                where=f"layer={l} b={b}")


def test_group_matches_standalone_calls_and_oracle():
    wl = _group_case()
    say(f"[indexshare_group_fwd] B={wl.B} T={wl.T} S={wl.S} k={wl.k} layers={wl.layers}")
    ind = synth.indexer_inputs(wl, device=DEV)
    layers = [synth.attention_inputs(wl, layer=l, device=DEV) for l in range(wl.layers)]
    args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    idx, outs, lses = bd.indexshare_group(*args, wl.k, [dict(q=L["q"], K=L["K"], V=L["V"])
                                                        for L in layers], wl.sm_scale,
                                          with_lse=True)
    # the same selection as a standalone ix_topk, the same outputs as standalone attention (300
    # query rows: the group's layers share the light kernel's launch, a standalone call runs
    # the other kernel, so within the split-rounding bound; bit for bit in the group attention)
    idx2 = bd.topk(*args, wl.k)
    assert torch.equal(idx, idx2)
    _same_as_group_attention(layers, idx, ind["kv_len"], wl.sm_scale, outs, lses)
    torch.cuda.synchronize()
    # and against the oracle: its own selection from the group's indexer, attention per layer
    h = to_host_indexer(ind)
    hl = [to_host_attn(L) for L in layers]
    idx_np = idx.cpu().numpy()
    for b in range(wl.B):
        keys = O.decode_e4m3(h["k_I"][b])
        ns = [O.visible_count(h["q_pos0"][b], h["kv_len"][b], t) for t in range(wl.T)]
        scs = [O.score_row(h["q_I"][b, t], keys[:ns[t]], h["w"][b, t], ns[t]) for t in range(wl.T)]
        ref_idx, same = oracle_selection(idx_np[b], scs, wl.k, ns, where=f"b={b}")
        assert same.mean() >= 0.9, f"b={b}: {int((~same).sum())} rows kept another tied set"
        for l in range(wl.layers):
            ref_o, ref_l = O.sparse_attention_rows(hl[l]["q"], hl[l]["K"], hl[l]["V"],
                                                   ref_idx, b, list(range(wl.T)), wl.sm_scale)
            check_attention(bf16_to_f64(outs[l])[b][same], ref_o[same],
                            lses[l].cpu().numpy()[b][same], ref_l[same], where=f"layer={l} b={b}")


def test_per_layer_baseline_with_identical_inputs_repeats_the_selection():
    wl = _group_case(B=1, T=64, S=2000, pos0s=None, kv_lens=None, pos0=1936, seed=42)
    ind = synth.indexer_inputs(wl, device=DEV)
    args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    say("[ix_topk x4] per-layer baseline")
    ref = bd.topk(*args, wl.k)
    for _ in range(3):
        assert torch.equal(bd.topk(*args, wl.k), ref)


def test_group_decode_shape():
    wl = _group_case(B=16, T=1, S=20000, pos0s=None, kv_lens=None, pos0=19999, k=2048, seed=43,
                     planted=32)
    say(f"[indexshare_group_fwd] decode B={wl.B} S={wl.S}")
    ind = synth.indexer_inputs(wl, device=DEV)
    layers = [synth.attention_inputs(wl, layer=l, device=DEV) for l in range(wl.layers)]
    args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    idx, outs, lses = bd.indexshare_group(*args, wl.k, [dict(q=L["q"], K=L["K"], V=L["V"])
                                                        for L in layers], wl.sm_scale,
                                          with_lse=True)
    # the layers share one attention launch: bit for bit sparse_attn_group_fwd on the same
    # selection, and standalone calls up to the rounding of the split merges
    _same_as_group_attention(layers, idx, ind["kv_len"], wl.sm_scale, outs, lses)
    torch.cuda.synchronize()
    h = to_host_indexer(ind)
    idx_np = idx.cpu().numpy()
    for b in range(0, wl.B, 3):
        keys = O.decode_e4m3(h["k_I"][b])
        n = O.visible_count(h["q_pos0"][b], h["kv_len"][b], 0)
        sc = O.score_row(h["q_I"][b, 0], keys[:n], h["w"][b, 0], n)
        ref_idx, same = oracle_selection(idx_np[b, :1], [sc], wl.k, [n], where=f"b={b}")
        if not same[0]:
            continue  # an equally valid tied set, checked above
        for l in range(wl.layers):
            hl = to_host_attn(layers[l])
            ref_o, _ = O.sparse_attention_rows(hl["q"], hl["K"], hl["V"], ref_idx, b, [0],
                                               wl.sm_scale)
            check_attention(bf16_to_f64(outs[l])[b], ref_o, where=f"layer={l} b={b}")


def test_group_of_ten_layers_decode_two_launches():
    """More layers than one launch takes (8): the attention runs as 8 + 2, bit for bit
    sparse_attn_group_fwd and standalone calls up to the rounding of split merges."""
    wl = _group_case(B=4, T=1, S=5000, pos0s=None, kv_lens=None, pos0=4999, k=512, seed=44,
                     layers=10, planted=16)
    say(f"[indexshare_group_fwd] decode B={wl.B} S={wl.S} layers={wl.layers}")
    ind = synth.indexer_inputs(wl, device=DEV)
    layers = [synth.attention_inputs(wl, layer=l, device=DEV) for l in range(wl.layers)]
    args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    idx, outs, lses = bd.indexshare_group(*args, wl.k, [dict(q=L["q"], K=L["K"], V=L["V"])
                                                        for L in layers], wl.sm_scale,
                                          with_lse=True)
    assert torch.equal(idx, bd.topk(*args, wl.k))
    _same_as_group_attention(layers, idx, ind["kv_len"], wl.sm_scale, outs, lses)
    torch.cuda.synchronize()
