"""GPU parity: indexer scores (ix_score) and the fused top-k (ix_topk) vs the oracle."""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from indexed_sparse_attention_ix_amd.workloads import WORKLOADS, Workload
from oracle import ix_oracle as O
from parity_util import (check_index_row, check_scores, say, score_magnitude, score_tolerance,
                         to_host_indexer)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _wl(**kw):
    base = dict(name="case", B=1, T=64, S=64, pos0=0, H_I=64, d_I=128, k=64, H_q=16, H_kv=1,
                d=128, layers=1, seed=11, qkv_std=1.0)
    base.update(kw)
    return Workload(**base)


def _run_scores(wl, t_begin=0, t_end=None, tweak=None):
    say(f"[ix_score] {wl.name} B={wl.B} T={wl.T} S={wl.S} H_I={wl.H_I} d_I={wl.d_I} seed={wl.seed}")
    ind = synth.indexer_inputs(wl, device=DEV)
    if tweak:
        tweak(ind)
    t_end = wl.T if t_end is None else t_end
    sc = bd.score(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"], t_begin, t_end)
    torch.cuda.synchronize()
    h = to_host_indexer(ind)
    for b in range(wl.B):
        rows = list(range(t_begin, t_end))
        ref = O.score_matrix(h["q_I"], h["k_I"], h["w"], h["q_pos0"], h["kv_len"], b, rows, wl.S)
        kabs = np.abs(O.decode_e4m3(h["k_I"][b]))
        mag = np.stack([score_magnitude(h["q_I"][b, t], kabs, h["w"][b, t]) for t in rows])
        check_scores(sc[b].cpu().numpy(), ref, mag, wl.d_I, wl.H_I)


def test_score_tiny_all_rows():
    _run_scores(WORKLOADS["tiny_prefill_1k"])


def test_score_ragged_lengths_and_head_counts():
    # kv_len below the query positions, a sequence whose queries outrun its cache,
    # 12 heads (3 MFMA column blocks), ragged tails on every tile size
    wl = _wl(B=2, T=77, S=300, pos0s=(100, 0), kv_lens=(250, 60), H_I=12, d_I=128, seed=12)
    _run_scores(wl, 5, 70)
    wl2 = _wl(B=1, T=45, S=133, pos0=88, H_I=8, d_I=64, seed=13)
    _run_scores(wl2)


def _run_topk(wl, check_sel=True, tweak=None):
    say(f"[ix_topk] {wl.name} B={wl.B} T={wl.T} S={wl.S} H_I={wl.H_I} d_I={wl.d_I} k={wl.k} "
        f"seed={wl.seed}")
    ind = synth.indexer_inputs(wl, device=DEV)
    if tweak:
        tweak(ind)
    idx, sel = bd.topk(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"], wl.k,
                       with_scores=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    sel = sel.cpu().numpy()
    h = to_host_indexer(ind)
    swaps = 0
    for b in range(wl.B):
        keys = O.decode_e4m3(h["k_I"][b])
        for t in range(wl.T):
            n = O.visible_count(h["q_pos0"][b], h["kv_len"][b], t)
            sc = O.score_row(h["q_I"][b, t], keys[:n], h["w"][b, t], n)
            swaps += check_index_row(idx[b, t], sc, wl.k, n, where=f"b={b} t={t}")
            if check_sel:
                m = min(wl.k, n)
                g = sel[b, t, :m].astype(np.float64)
                r = sc[idx[b, t, :m]]
                mag = score_magnitude(h["q_I"][b, t], np.abs(keys[idx[b, t, :m]]), h["w"][b, t])
                assert np.all(np.abs(g - r) <= score_tolerance(r, mag, wl.d_I, wl.H_I))
                assert np.all(np.isneginf(sel[b, t, m:]))
    say(f"  swaps inside the tie band: {swaps}")
    return idx


def _flip_every_third_head(ind):
    H = ind["w"].shape[-1]
    sign = torch.where(torch.arange(H, device=ind["w"].device) % 3 == 0, -1.0, 1.0)
    ind["w"] = (ind["w"] * sign).contiguous()


def test_mixed_sign_head_weights():
    """Head weights of both signs at 64 heads (scores may be negative; keys whose heads are
    all <= 0 still score exactly 0), through ix_score and the fused top-k with and without a
    threshold sample."""
    wl = _wl(B=2, T=40, S=700, pos0s=(660, 300), kv_lens=(700, 500), seed=31)
    _run_scores(wl, tweak=_flip_every_third_head)
    _run_topk(wl, tweak=_flip_every_third_head)
    wl2 = _wl(B=1, T=9, S=9000, pos0=8991, k=256, seed=32, planted=8)
    _run_topk(wl2, tweak=_flip_every_third_head)


def test_topk_tiny_all_rows():
    _run_topk(WORKLOADS["tiny_prefill_1k"])


def test_topk_buffer_compaction_ragged():
    # visible prefixes far beyond the candidate capacity (several compactions per query),
    # ragged kv_len, queries not a multiple of the wave's 4
    wl = _wl(B=2, T=203, S=6000, pos0s=(5797, 2000), kv_lens=(6000, 4100), H_I=64, k=300,
             seed=14, planted=8)
    _run_topk(wl)


def test_topk_key_splits_and_merge():
    # one query per sequence: one query per wave, keys split over several waves, merged
    wl = _wl(B=5, T=1, S=40000, pos0=39999, H_I=64, k=2048, seed=15, planted=32)
    _run_topk(wl)
    wl2 = _wl(B=3, T=2, S=20000, pos0=19998, H_I=16, d_I=64, k=100, seed=16)
    _run_topk(wl2)


def _run_topk_concentrated(wl, hot_keys):
    """Scale the first `hot_keys` indexer keys by 2 so that nearly the whole top-k sits in
    the first key split: more than that split keeps, so the merge cannot prove its union
    and the query takes the recompute pass (every split keeping its exact top-k)."""
    say(f"[ix_topk] concentrated top-k B={wl.B} T={wl.T} S={wl.S} k={wl.k} hot={hot_keys}")
    ind = synth.indexer_inputs(wl, device=DEV)
    kf = synth.decode_e4m3_torch(ind["k_I"])
    kf[:, :hot_keys] *= 2.0
    ind["k_I"] = synth.encode_e4m3(kf)
    idx, sel = bd.topk(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"], wl.k,
                       with_scores=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    h = to_host_indexer(ind)
    for b in range(wl.B):
        keys = O.decode_e4m3(h["k_I"][b])
        for t in range(wl.T):
            n = O.visible_count(h["q_pos0"][b], h["kv_len"][b], t)
            sc = O.score_row(h["q_I"][b, t], keys[:n], h["w"][b, t], n)
            check_index_row(idx[b, t], sc, wl.k, n, where=f"b={b} t={t}")
            assert (idx[b, t, : wl.k] < hot_keys).sum() > wl.k // 2  # the case it is meant to be


def test_topk_split_union_unproven_takes_recompute_pass():
    # one query per wave (16 heads per MFMA column block) and four per wave
    _run_topk_concentrated(_wl(B=2, T=1, S=65536, pos0=65535, k=2048, seed=19, qkv_std=1.0), 4096)
    _run_topk_concentrated(_wl(B=1, T=4, S=65536, pos0=65532, k=2048, seed=20, qkv_std=1.0), 4096)


def test_topk_sampled_threshold_all_rows():
    # long enough prefixes (>= 4 tiles per sampled tile) for the starting-threshold sample;
    # the second sequence's prefixes are too short for it
    wl = _wl(B=2, T=37, S=8000, pos0s=(7963, 5000), H_I=64, k=256, seed=22, planted=8)
    _run_topk(wl)


def _sample_tiles(n_keys, k, pf=2):
    """Stride and tiles of the starting-threshold sample for one unsplit query group with
    16 MFMA head blocks: at most 64 tiles (they must fit a candidate buffer), one per
    stride group, picked inside group jj by the multiplicative hash the kernel uses."""
    kpad = (k + 63) // 64 * 64
    stage = 2 * 64 * pf
    cap = 2 * kpad + max(1024, 2 * stage)
    samp = min(64, (cap - stage) // 16)
    stride = ((n_keys + 15) // 16) // samp
    tiles = [stride * jj + (((jj * 2654435761) % (1 << 32)) >> 16) % stride for jj in range(samp)]
    return stride, tiles


def test_topk_misleading_sample_takes_second_sweep():
    """The sampled tiles get doubled keys, so the sampled threshold sits far above the
    true k-th score: too few keys pass and the wave must sweep again from zero."""
    wl = _wl(B=1, T=4, S=8000, pos0=7996, H_I=64, k=256, seed=23)
    stride, sampled = _sample_tiles(8000, wl.k)
    assert stride >= 4
    say(f"[ix_topk] misleading sample, stride {stride}")
    ind = synth.indexer_inputs(wl, device=DEV)
    kf = synth.decode_e4m3_torch(ind["k_I"])
    tiles = torch.arange(wl.S, device=DEV) // 16
    kf[:, torch.isin(tiles, torch.tensor(sampled, device=DEV))] *= 2.0
    ind["k_I"] = synth.encode_e4m3(kf)
    idx = bd.topk(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"], wl.k)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    h = to_host_indexer(ind)
    keys = O.decode_e4m3(h["k_I"][0])
    for t in range(wl.T):
        n = O.visible_count(h["q_pos0"][0], h["kv_len"][0], t)
        sc = O.score_row(h["q_I"][0, t], keys[:n], h["w"][0, t], n)
        check_index_row(idx[0, t], sc, wl.k, n, where=f"t={t}")


def test_topk_k_at_least_visible_keeps_everything():
    wl = _wl(B=1, T=40, S=50, pos0=10, H_I=4, d_I=64, k=64, seed=17)
    idx = _run_topk(wl)
    for t in range(wl.T):
        n = min(10 + t + 1, 50)
        assert idx[0, t, :n].tolist() == list(range(n))


def _e4m3_code(v):
    return int(np.nonzero(O.E4M3_TABLE == v)[0][0])


@pytest.mark.parametrize("H,S,mixed", [(8, 3000, False), (64, 3000, False), (64, 20000, False),
                                       (64, 3000, True)])
def test_topk_known_top_set_with_zero_ties(H, S, mixed):
    """Queries >= 0 and unplanted keys <= 0 give exact zero scores; planted keys have
    closed-form distinct scores.  The kept set is known exactly (no tie band).  With 64
    heads the scores come from the |x| + linear-MFMA form, whose zero keys are rescored
    (20000 keys: also after a threshold sample; mixed: every third head weight is -1)."""
    rng = np.random.default_rng(21)
    B, T, d, k = 2, 8, 128, 100
    neg = [c for c in range(256) if O.E4M3_TABLE[c] <= 0 and not np.isnan(O.E4M3_TABLE[c])]
    kc = rng.choice(neg, size=(B, S, d)).astype(np.uint8)
    vals = [0.5 + 0.0625 * i for i in range(8)] + [1.0 + 0.125 * i for i in range(8)]
    planted = {}
    for b in range(B):
        pos = sorted(rng.choice(np.arange(S), size=len(vals), replace=False).tolist())
        v = list(vals)
        rng.shuffle(v)
        planted[b] = dict(zip(pos, v))
        for s, x in planted[b].items():
            kc[b, s, :] = _e4m3_code(x)
    qc = np.full((B, T, H, d), _e4m3_code(0.25), dtype=np.uint8)
    w = np.ones((B, T, H), dtype=np.float32)
    if mixed:
        w[..., ::3] = -1.0
    pos0 = np.array([S - T, 1500], dtype=np.int32)
    kvl = np.array([S, S], dtype=np.int32)
    dev = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    say("[ix_topk] sign-partitioned planting")
    idx = bd.topk(dev(qc), dev(kc), dev(w), dev(pos0), dev(kvl), k).cpu().numpy()
    for b in range(B):
        for t in range(T):
            n = min(int(pos0[b]) + t + 1, S)
            vis = {s: x for s, x in planted[b].items() if s < n}
            order = sorted(vis, key=lambda s: -vis[s])[:k]
            zeros = [s for s in range(n) if s not in vis][: k - len(order)]
            assert idx[b, t].tolist() == sorted(order + zeros), f"b={b} t={t}"
    # every score is exact here: 0 for the unplanted keys, H * d * 0.25 * x for planted ones
    sc = bd.score(dev(qc), dev(kc), dev(w), dev(pos0), dev(kvl)).cpu().numpy()
    for b in range(B):
        for t in range(T):
            n = min(int(pos0[b]) + t + 1, S)
            want = np.zeros(n, dtype=np.float32)
            for s, x in planted[b].items():
                if s < n:
                    want[s] = w[b, t].sum() * d * 0.25 * x
            assert np.array_equal(sc[b, t, :n], want), f"scores b={b} t={t}"


def test_topk_is_deterministic():
    wl = _wl(B=1, T=64, S=9000, pos0=8936, k=512, seed=18)
    ind = synth.indexer_inputs(wl, device=DEV)
    say("[ix_topk] determinism")
    a = bd.topk(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"], wl.k)
    b = bd.topk(ind["q_I"], ind["k_I"], ind["w"], ind["q_pos0"], ind["kv_len"], wl.k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
