"""GPU parity: sparse attention (sparse_attn_fwd) vs the oracle on the same index tensor."""
import math

import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from indexed_sparse_attention_ix_amd.workloads import WORKLOADS, Workload
from oracle import ix_oracle as O
from parity_util import bf16_to_f64, check_attention, say, to_host_attn

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _wl(**kw):
    base = dict(name="attn", B=1, T=64, S=64, pos0=0, H_I=4, d_I=64, k=64, H_q=16, H_kv=1, d=128,
                layers=1, seed=31, qkv_std=1.0 / math.sqrt(128))
    base.update(kw)
    return Workload(**base)


def _random_idx(wl, rng, frac_pad=0.1):
    """Ascending distinct visible positions with some -1 padding per row."""
    idx = np.full((wl.B, wl.T, wl.k), -1, dtype=np.int32)
    for b in range(wl.B):
        for t in range(wl.T):
            n = wl.visible(b, t)
            m = min(wl.k, n)
            if m > 1 and rng.random() < frac_pad:
                m = int(rng.integers(1, m))
            idx[b, t, :m] = np.sort(rng.choice(n, size=m, replace=False))
    return idx


def _run_attn(wl, idx_np, att=None, sm_scale=None, tag=""):
    say(f"[sparse_attn_fwd] {tag} B={wl.B} T={wl.T} S={wl.S} H_q={wl.H_q} H_kv={wl.H_kv} "
        f"d={wl.d} k={wl.k} seed={wl.seed}")
    att = att if att is not None else synth.attention_inputs(wl, device=DEV)
    sm = wl.sm_scale if sm_scale is None else sm_scale
    kvl = torch.tensor(wl.kv_len_list(), dtype=torch.int32, device=DEV)
    idx = torch.from_numpy(idx_np).to(DEV)
    out, lse = bd.sparse_attention(att["q"], att["K"], att["V"], idx, sm, kv_len=kvl,
                                   with_lse=True)
    torch.cuda.synchronize()
    h = to_host_attn(att)
    og = bf16_to_f64(out)
    lg = lse.cpu().numpy().astype(np.float64)
    # entries past kv_len / S_max are padding by contract: the oracle sees them as -1
    kv = np.array(wl.kv_len_list())[:, None, None]
    ref_idx = np.where((idx_np >= kv) | (idx_np >= wl.S), -1, idx_np)
    for b in range(wl.B):
        ref_o, ref_l = O.sparse_attention_rows(h["q"], h["K"], h["V"], ref_idx[b], b,
                                               list(range(wl.T)), sm)
        check_attention(og[b], ref_o, lg[b], ref_l, where=f"{tag} b={b}")
    return out, lse


def test_attention_tiny_with_oracle_selection():
    wl = WORKLOADS["tiny_prefill_1k"]
    ind = synth.indexer_inputs(wl)  # host generation; selection from the oracle
    h = {k: v.numpy() for k, v in ind.items()}
    idx = O.topk_rows(h["q_I"], h["k_I"], h["w"], h["q_pos0"], h["kv_len"], 0,
                      list(range(wl.T)), wl.k).astype(np.int32)[None]
    _run_attn(wl, idx, tag="tiny")


def test_attention_full_selection_is_dense_causal():
    wl = _wl(T=200, S=200, k=256, d=64, H_q=8, seed=32, qkv_std=1.0)
    idx = np.full((1, wl.T, wl.k), -1, dtype=np.int32)
    for t in range(wl.T):
        idx[0, t, : t + 1] = np.arange(t + 1)
    out, lse = _run_attn(wl, idx, tag="dense")
    # and against torch's SDPA in fp32 on the CPU (a library routine, not the oracle)
    att = synth.attention_inputs(wl, device=DEV)
    q = att["q"].float().cpu()[0].permute(1, 0, 2)
    K = att["K"].float().cpu()[0].permute(1, 0, 2).expand(wl.H_q, -1, -1)
    V = att["V"].float().cpu()[0].permute(1, 0, 2).expand(wl.H_q, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, is_causal=True,
                                                           scale=wl.sm_scale)
    g = out.float().cpu()[0].permute(1, 0, 2)
    assert (g - ref).abs().max().item() < 2e-2


def test_attention_k1_returns_the_selected_row():
    wl = _wl(B=2, T=50, S=300, pos0=250, k=1, seed=33)
    rng = np.random.default_rng(33)
    idx = _random_idx(wl, rng, frac_pad=0.0)
    att = synth.attention_inputs(wl, device=DEV)
    out, _ = _run_attn(wl, idx, att=att, tag="k=1")
    V = att["V"].cpu()
    for b in range(wl.B):
        for t in range(wl.T):
            row = V[b, idx[b, t, 0], 0]
            assert torch.equal(out[b, t].cpu(), row[None, :].expand(wl.H_q, -1))


def test_attention_sharp_logits_and_padding():
    # q scaled so that logits have std ~4: softmax is peaked, so a wrong row shows
    wl = _wl(B=1, T=96, S=5000, pos0=4904, k=700, seed=34)
    att = synth.attention_inputs(wl, device=DEV)
    att["q"] = (att["q"].float() * (4.0 * math.sqrt(wl.d) * math.sqrt(wl.d))).to(torch.bfloat16)
    rng = np.random.default_rng(34)
    idx = _random_idx(wl, rng, frac_pad=0.3)
    idx[0, 3, :] = -1            # empty selection: out = 0, lse = -inf
    idx[0, 4, 10] = 4999 + 50    # beyond kv_len: skipped
    idx[0, 4, 11] = 1 << 30      # beyond S_max: skipped
    _run_attn(wl, idx, att=att, tag="sharp")


def test_attention_gqa_and_small_head_dim():
    wl = _wl(B=2, T=33, S=500, pos0=467, k=130, H_q=16, H_kv=2, d=64, seed=35, qkv_std=1.0)
    rng = np.random.default_rng(35)
    _run_attn(wl, _random_idx(wl, rng), tag="gqa")


def test_attention_decode_split_path():
    # 64 single-token queries: the selection is split over several blocks per query
    wl = _wl(B=64, T=1, S=6000, pos0=5999, k=2048, seed=36)
    assert bd.sparse_attn_workspace_bytes(wl.B, wl.T, wl.H_q, wl.H_kv, wl.d, wl.k) > 0
    rng = np.random.default_rng(36)
    _run_attn(wl, _random_idx(wl, rng), tag="decode")


def test_attention_is_deterministic():
    wl = _wl(B=1, T=128, S=4000, pos0=3872, k=1024, seed=37)
    rng = np.random.default_rng(37)
    idx = torch.from_numpy(_random_idx(wl, rng)).to(DEV)
    att = synth.attention_inputs(wl, device=DEV)
    say("[sparse_attn_fwd] determinism")
    a = bd.sparse_attention(att["q"], att["K"], att["V"], idx, wl.sm_scale)
    b = bd.sparse_attention(att["q"], att["K"], att["V"], idx, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# Grids of 1024 query rows (B * T * H_kv) or more take the main kernel (32-entry chunks staged
# in LDS); the cases above, all smaller, take the light kernel.  These repeat the awkward
# shapes there: a selection length that is not a whole number of chunks (nor of 4 entries),
# grouped heads with d = 64, padding, empty rows, entries past kv_len and S_max, k = 1.
@pytest.mark.parametrize("case", ["ragged_gqa_d64", "sharp_padding", "k1", "two_sequences"])
def test_attention_main_kernel_shapes(case):
    if case == "ragged_gqa_d64":
        wl = _wl(B=1, T=520, S=1500, pos0=980, k=130, H_q=16, H_kv=2, d=64, seed=41, qkv_std=1.0)
    elif case == "sharp_padding":
        wl = _wl(B=1, T=1030, S=3000, pos0=1970, k=301, seed=42)
    elif case == "k1":
        wl = _wl(B=2, T=520, S=2000, pos0=1480, k=1, seed=43)
    else:
        wl = _wl(B=2, T=600, S=3000, pos0=2400, k=37, H_q=8, seed=44)
    assert wl.B * wl.T * wl.H_kv >= 1024
    rng = np.random.default_rng(wl.seed)
    idx = _random_idx(wl, rng, frac_pad=0.0 if case == "k1" else 0.3)
    att = synth.attention_inputs(wl, device=DEV)
    if case == "sharp_padding":
        att["q"] = (att["q"].float() * (4.0 * wl.d)).to(torch.bfloat16)
        idx[0, 3, :] = -1
        idx[0, 4, 10] = wl.S + 50
        idx[0, 4, 11] = 1 << 30
    out, _ = _run_attn(wl, idx, att=att, tag="main " + case)
    if case == "k1":
        V = att["V"].cpu()
        for b in range(wl.B):
            for t in range(0, wl.T, 7):
                row = V[b, idx[b, t, 0], 0]
                assert torch.equal(out[b, t].cpu(), row[None, :].expand(wl.H_q, -1))
