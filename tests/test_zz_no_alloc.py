"""indexshare_group_fwd_noalloc (the group forward on the library's own scratch, for callers
that cannot allocate) against indexshare_group_fwd with a caller workspace, through the C ABI:
two calls in a row, the second on a smaller input, and the size limit."""
import math

import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from indexed_sparse_attention_ix_amd.workloads import Workload
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(**kw):
    base = dict(name="noalloc", B=1, T=1, S=4096, pos0=0, H_I=64, d_I=128, k=2048, H_q=16,
                H_kv=1, d=128, layers=4, seed=61, qkv_std=1.0 / math.sqrt(128), planted=8)
    base.update(kw)
    return Workload(**base)


def _inputs(wl):
    ind = synth.indexer_inputs(wl, device=DEV)
    layers = [synth.attention_inputs(wl, layer=l, device=DEV) for l in range(wl.layers)]
    a = bd.indexer_args(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"])
    return ind, layers, a


def _group(wl, a, layers, noalloc):
    """One group call through the C ABI; returns idx, outputs and lse per layer."""
    idx = torch.full((wl.B, wl.T, wl.k), -7, dtype=torch.int32, device=DEV)
    outs = [torch.full_like(L["q"], 3.0) for L in layers]
    lses = [torch.full((wl.B, wl.T, wl.H_q), 5.0, dtype=torch.float32, device=DEV) for _ in layers]
    ptrs = ([L["q"].data_ptr() for L in layers], [L["K"].data_ptr() for L in layers],
            [L["V"].data_ptr() for L in layers], [o.data_ptr() for o in outs],
            [x.data_ptr() for x in lses])
    sh = torch.cuda.current_stream().cuda_stream
    if noalloc:
        bd.indexshare_group_fwd_noalloc(a, wl.k, wl.layers, *ptrs, wl.H_q, wl.H_kv, wl.d,
                                        wl.sm_scale, idx.data_ptr(), sh)
    else:
        nb = bd.indexshare_workspace_bytes(a, wl.k, wl.H_q, wl.H_kv, wl.d)
        ws = torch.full((max(nb, 256),), 0xFF, dtype=torch.uint8, device=DEV)  # stale contents
        bd.indexshare_group_fwd(a, wl.k, wl.layers, *ptrs, wl.H_q, wl.H_kv, wl.d, wl.sm_scale,
                                idx.data_ptr(), ws.data_ptr(), nb, sh)
    torch.cuda.synchronize()
    return idx, outs, lses


def test_noalloc_matches_workspace_entry_point_twice():
    # a decode step (key splits, merge, split attention, the layers in one launch), then a
    # smaller ragged prefill: each bitwise equal to indexshare_group_fwd with a workspace
    cases = [_case(B=24, T=1, S=65536, pos0=65535, layers=4, seed=61),
             _case(B=2, T=150, S=1500, pos0=0, pos0s=(1350, 400), kv_lens=(1500, 1200), k=256,
                   layers=2, seed=62)]
    for i, wl in enumerate(cases):
        ind, layers, a = _inputs(wl)
        need = bd.indexshare_workspace_bytes(a, wl.k, wl.H_q, wl.H_kv, wl.d)
        say(f"[noalloc call {i}] B={wl.B} T={wl.T} S={wl.S} k={wl.k} layers={wl.layers} "
            f"workspace {need} bytes")
        assert 0 < need <= bd.NOALLOC_SCRATCH_BYTES
        got = _group(wl, a, layers, noalloc=True)
        ref = _group(wl, a, layers, noalloc=False)
        assert torch.equal(got[0], ref[0]), f"call {i}: idx differs"
        for l in range(wl.layers):
            assert torch.equal(got[1][l], ref[1][l]), f"call {i} layer {l}: out differs"
            assert torch.equal(got[2][l], ref[2][l]), f"call {i} layer {l}: lse differs"
        # the selection is a real one: ascending, distinct, visible
        idx = got[0].cpu()
        for b in range(wl.B):
            for t in range(wl.T):
                row = idx[b, t]
                v = row[row >= 0]
                assert len(v) == min(wl.k, wl.visible(b, t))
                assert bool((v[1:] > v[:-1]).all()) and int(v.max()) < wl.visible(b, t)


def test_noalloc_rejects_calls_beyond_its_scratch():
    wl = _case(B=1, T=2048, S=2048, k=2048, layers=1, seed=63)
    ind, layers, a = _inputs(wl)
    need = bd.indexshare_workspace_bytes(a, wl.k, wl.H_q, wl.H_kv, wl.d)
    assert need > bd.NOALLOC_SCRATCH_BYTES
    with pytest.raises(bd.IxError) as e:
        _group(wl, a, layers, noalloc=True)
    assert e.value.status == bd.IX_ERR_WORKSPACE and "scratch" in str(e.value)
