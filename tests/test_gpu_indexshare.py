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


def test_group_matches_standalone_calls_bitwise_and_oracle():
    wl = _group_case()
    say(f"[indexshare_group_fwd] B={wl.B} T={wl.T} S={wl.S} k={wl.k} layers={wl.layers}")
    ind = synth.indexer_inputs(wl, device=DEV)
    layers = [synth.attention_inputs(wl, layer=l, device=DEV) for l in range(wl.layers)]
    args = (ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    idx, outs, lses = bd.indexshare_group(*args, wl.k, [dict(q=L["q"], K=L["K"], V=L["V"])
                                                        for L in layers], wl.sm_scale,
                                          with_lse=True)
    # the same selection as a standalone ix_topk, the same outputs as standalone attention
    idx2 = bd.topk(*args, wl.k)
    assert torch.equal(idx, idx2)
    for l, L in enumerate(layers):
        o2, l2 = bd.sparse_attention(L["q"], L["K"], L["V"], idx, wl.sm_scale,
                                     kv_len=ind["kv_len"], with_lse=True)
        assert torch.equal(outs[l], o2) and torch.equal(lses[l], l2)
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
    # the layers share one attention launch (split partials per layer, one combine): the
    # same bits as standalone calls
    for l, L in enumerate(layers):
        o2, l2 = bd.sparse_attention(L["q"], L["K"], L["V"], idx, wl.sm_scale,
                                     kv_len=ind["kv_len"], with_lse=True)
        assert torch.equal(outs[l], o2) and torch.equal(lses[l], l2), f"layer {l}"
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
    """More layers than one launch takes (8): the attention runs as 8 + 2, still bit for bit
    the standalone calls."""
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
    for l, L in enumerate(layers):
        o2, l2 = bd.sparse_attention(L["q"], L["K"], L["V"], idx, wl.sm_scale,
                                     kv_len=ind["kv_len"], with_lse=True)
        assert torch.equal(outs[l], o2) and torch.equal(lses[l], l2), f"layer {l}"
    torch.cuda.synchronize()
