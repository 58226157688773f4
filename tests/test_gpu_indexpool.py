"""GPU parity: IndexPool's block keys (ix_pool_keys, bit-exact) and the block selection
expanded to tokens (ix_topk_pooled) against the oracle."""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from indexed_sparse_attention_ix_amd.workloads import Workload
from oracle import ix_oracle as O
from parity_util import check_index_row, say, to_host_indexer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _wl(**kw):
    base = dict(name="pool_case", B=1, T=16, S=1000, pos0=0, H_I=64, d_I=128, k=256, H_q=16,
                H_kv=1, d=128, layers=1, seed=51, qkv_std=1.0)
    base.update(kw)
    return Workload(**base)


def test_pool_keys_bit_exact():
    for d_I, S, kvl, pool in ((128, 1001, [1001, 503], 4), (64, 77, [70, 0], 2), (128, 64, [64, 61], 16)):
        say(f"[ix_pool_keys] d_I={d_I} S={S} kv_len={kvl} pool={pool}")
        g = torch.Generator(device="cpu").manual_seed(52 + d_I + S)
        codes = torch.randint(0, 256, (2, S, d_I), generator=g, dtype=torch.int32).to(torch.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x38   # a cache holds no NaN codes
        kv = torch.tensor(kvl, dtype=torch.int32)
        got = bd.pool_keys(codes.to(DEV), kv.to(DEV), pool).cpu().numpy()
        for b in range(2):
            want = O.pool_keys(codes[b].numpy(), kvl[b], pool)
            assert np.array_equal(got[b], want), (d_I, S, b)


def _run_pooled(wl, pool, k_blocks):
    say(f"[ix_topk_pooled] B={wl.B} T={wl.T} S={wl.S} pool={pool} k_blocks={k_blocks} seed={wl.seed}")
    ind = synth.indexer_inputs(wl, device=DEV)
    kp = bd.pool_keys(ind["k_I"], ind["kv_len"], pool)
    idx = bd.topk_pooled(ind["q_I"], kp, ind["w"], ind["q_pos0"], ind["kv_len"], wl.S, pool,
                         k_blocks)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    h = to_host_indexer(ind)
    kp_h = kp.cpu().numpy()
    for b in range(wl.B):
        pooled_ref = O.pool_keys(h["k_I"][b], int(h["kv_len"][b]), pool)
        assert np.array_equal(kp_h[b], pooled_ref)
        pooled = O.decode_e4m3(pooled_ref)
        for t in range(wl.T):
            pos0, kvl = int(h["q_pos0"][b]), int(h["kv_len"][b])
            sc, _, _ = O.pooled_topk_row(h["q_I"][b, t], pooled, h["w"][b, t], pos0, kvl, t,
                                         pool, k_blocks)
            row = idx[b, t]
            # the kept blocks (every kept block shows at least its first token)
            blocks = sorted(set((row[row >= 0] // pool).tolist()))
            padded = np.full(k_blocks, -1, dtype=np.int64)
            padded[:len(blocks)] = blocks
            check_index_row(padded, sc, k_blocks, len(sc), where=f"b={b} t={t}")
            n_t = O.visible_count(pos0, kvl, t)
            toks = [pool * j + r for j in blocks for r in range(pool) if pool * j + r < n_t]
            want = np.full(k_blocks * pool, -1, dtype=np.int64)
            want[:len(toks)] = toks
            assert np.array_equal(row, want), f"expansion b={b} t={t}"


def test_topk_pooled_prefill_all_rows_ragged():
    wl = _wl(B=2, T=50, S=3000, pos0s=(2950, 1000), kv_lens=(3000, 1499), k=256, seed=53,
             planted=8)
    _run_pooled(wl, 4, 64)


def test_topk_pooled_decode_with_key_splits():
    # one query per sequence over 32768 blocks: split over several waves, each keeping
    # fewer than k_blocks, then merged
    wl = _wl(B=3, T=1, S=131072, pos0=131071, k=2048, seed=54, planted=32)
    _run_pooled(wl, 4, 512)


def test_topk_pooled_pool_1_matches_topk():
    wl = _wl(B=1, T=20, S=2000, pos0=1980, k=128, seed=55)
    ind = synth.indexer_inputs(wl, device=DEV)
    say("[ix_topk_pooled] pool 1 against ix_topk")
    kp = bd.pool_keys(ind["k_I"], ind["kv_len"], 1)
    a = bd.topk_pooled(ind["q_I"], kp, ind["w"], ind["q_pos0"], ind["kv_len"], wl.S, 1, wl.k)
    b = bd.topk(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"], wl.k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
