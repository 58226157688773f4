"""GPU parity: the indexer backward (ix_indexer_bwd) against the oracle, every entry.

Tolerance, per entry, against B = the same gradient computed by the oracle on absolute
values (|q_I|, |k_I|, |w|, |dscores|), which bounds the sum of the magnitudes of the terms.
The MFMAs (FP8 for the dot products, bf16 for the two products) accumulate more coarsely
than fp32: their error, measured up to 7e-5 of the sum of the magnitudes, is bounded here
by M = 2^-13 (independent of the depth).  With u = 2^-24:
  dw:   M B from the dot products, plus k fp32 additions: (M + (k + 2) u) B.
  dq:   d loss / d x enters the bf16 products as a hi + lo pair (residual <= 2^-18 = 64 u);
        the products of e4m3 values are exact: (M + (64 + k) u) B.
  dk:   the same per query, plus one fp32 atomic addition per query that kept the key:
        (M + (64 + T) u) B.
The ReLU mask is exact on both sides (the oracle's dot products are exact; the kernel
recomputes exactly any dot product within 2^-10 |q| |k| of zero, 8x above M), so a flipped
mask, which moves an entry by about B / k, cannot pass.
"""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from oracle import ix_oracle as O
from parity_util import abs_codes, check_indexer_bwd, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(qI, kI, w, kvl, idx, ds, rows_per_pass=None, pair_rows=bd.PAIR_ROWS_BF16):
    B, T, H, d_I = qI.shape
    t = {n: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
         for n, v in (("q", qI), ("k", kI), ("w", w.astype(np.float32)),
                      ("kvl", kvl.astype(np.int32)), ("idx", idx.astype(np.int32)),
                      ("ds", ds.astype(np.float32)))}
    pos0 = torch.zeros(B, dtype=torch.int32, device=DEV)
    args = bd.indexer_args(t["q"], t["k"], t["w"], pos0, t["kvl"])
    dq, dw, dk = bd.indexer_bwd(args, t["idx"], t["ds"], DEV, rows_per_pass=rows_per_pass,
                                pair_rows=pair_rows)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dw.cpu().numpy(), dk.cpu().numpy()


def _case(seed, B, T, S, H, d_I, k, kv_lens, values=None, empty_rows=(), past_kv=0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    if values is None:
        qI = synth.encode_e4m3(torch.randn(B, T, H, d_I, generator=g) * 2).numpy()
        kI = synth.encode_e4m3(torch.randn(B, S, d_I, generator=g)).numpy()
    else:
        vals = torch.tensor(values, dtype=torch.float32)
        qI = synth.encode_e4m3(vals[torch.randint(len(values), (B, T, H, d_I), generator=g)]).numpy()
        kI = synth.encode_e4m3(vals[torch.randint(len(values), (B, S, d_I), generator=g)]).numpy()
    w = torch.randn(B, T, H, generator=g).numpy().astype(np.float32)
    rng = np.random.default_rng(seed)
    kvl = np.array(kv_lens, dtype=np.int32)
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            if (b, t) in empty_rows:
                continue
            hi = min(S, int(kvl[b]) + past_kv)        # some entries past kv_len: padding
            if hi == 0:
                continue
            n = int(rng.integers(1, min(k, hi) + 1))
            idx[b, t, :n] = np.sort(rng.choice(hi, size=n, replace=False))
    ds = rng.standard_normal((B, T, k)).astype(np.float32)
    return qI, kI, w, kvl, idx, ds


# (rows_per_pass, pair_rows).  None: dk_I added with atomics; a row count: the atomic-free form
# (inverted selection, per-pair rows in bf16 or fp32, key-major sums) in passes of that many
# query rows
BF, F32 = bd.PAIR_ROWS_BF16, bd.PAIR_ROWS_FP32
MODES = [(None, BF), (1 << 20, BF), (7, BF), (1 << 20, F32), (7, F32)]


def _bf16_rows(rows_per_pass, pair_rows):
    return rows_per_pass is not None and pair_rows == BF


@pytest.mark.parametrize("rows_per_pass,pair_rows", MODES)
def test_indexer_bwd_ragged_64_heads_d128(rows_per_pass, pair_rows):
    say(f"[ix_indexer_bwd] B=2 T=40 S=500 H_I=64 d_I=128 k=96, ragged kv_len, empty row, "
        f"rows per pass {rows_per_pass}, pair rows {pair_rows}")
    qI, kI, w, kvl, idx, ds = _case(201, 2, 40, 500, 64, 128, 96, [500, 213], empty_rows={(1, 7)},
                                    past_kv=20)
    got = _run(qI, kI, w, kvl, idx, ds, rows_per_pass, pair_rows)
    assert np.all(got[0][1, 7] == 0) and np.all(got[1][1, 7] == 0)
    check_indexer_bwd(got, qI, kI, w, idx, ds, kvl, bf16_rows=_bf16_rows(rows_per_pass, pair_rows))


@pytest.mark.parametrize("rows_per_pass,pair_rows", MODES)
def test_indexer_bwd_exact_zero_dots_partial_head_tile_d64(rows_per_pass, pair_rows):
    """Codes in {0, +-1, +-2}: many dot products are exactly 0 (gradient 0 there on both
    sides); 20 heads leave a partial tile of 16; k = 37 leaves a ragged chunk."""
    say(f"[ix_indexer_bwd] B=1 T=33 S=300 H_I=20 d_I=64 k=37, integer codes, rows per pass "
        f"{rows_per_pass}, pair rows {pair_rows}")
    qI, kI, w, kvl, idx, ds = _case(202, 1, 33, 300, 20, 64, 37, [300],
                                    values=[0.0, 0.0, 0.0, 1.0, -1.0, 2.0, -2.0])
    keys = O.decode_e4m3(kI[0])
    x0 = O.decode_e4m3(qI[0]) @ keys.T
    say(f"  exact zero dot products: {int((x0 == 0).sum())} of {x0.size}")
    assert (x0 == 0).sum() > 100
    check_indexer_bwd(_run(qI, kI, w, kvl, idx, ds, rows_per_pass, pair_rows), qI, kI, w, idx, ds,
                      kvl, bf16_rows=_bf16_rows(rows_per_pass, pair_rows))


def test_indexer_bwd_full_k_and_few_heads():
    say("[ix_indexer_bwd] B=1 T=6 S=2300 H_I=4 d_I=128 k=2048")
    qI, kI, w, kvl, idx, ds = _case(203, 1, 6, 2300, 4, 128, 2048, [2300])
    check_indexer_bwd(_run(qI, kI, w, kvl, idx, ds), qI, kI, w, idx, ds, kvl)


def test_indexer_bwd_zero_dscores_and_all_padding():
    """dscores 0 everywhere gives zeros; a batch whose kv_len is 0 has only padding."""
    say("[ix_indexer_bwd] zero dscores, kv_len 0")
    qI, kI, w, kvl, idx, ds = _case(204, 2, 8, 100, 8, 64, 16, [100, 0], past_kv=10)
    dq, dw, dk = _run(qI, kI, w, kvl, idx, np.zeros_like(ds))
    assert not dq.any() and not dw.any() and not dk.any()
    dq, dw, dk = _run(qI, kI, w, kvl, idx, ds)
    assert not dq[1].any() and not dw[1].any() and not dk[1].any()
    check_indexer_bwd((dq, dw, dk), qI, kI, w, idx, ds, kvl)


def test_indexer_bwd_training_chain_exact_scores():
    """ix_topk -> sparse_attn_fwd (lse) -> ix_indexer_kl -> ix_indexer_bwd against the
    oracle's own chain.  Indexer codes in {0, +-0.5, +-1} and head weights that are
    multiples of 1/64 make every score exact in fp32, so both sides keep the same keys
    (ties to the lower index) with the same scores; the KL gradient differs by at most its
    own tolerance eps_j, whose effect on the indexer gradients is bounded by the oracle's
    backward on absolute values with dscores = eps."""
    B, T, S, H, d_I, k = 1, 48, 900, 16, 128, 128
    H_q, d, scale, temp = 8, 64, 64 ** -0.5, 0.25
    say(f"[ix_indexer_bwd] chain B={B} T={T} S={S} H_I={H} k={k}")
    g = torch.Generator(device="cpu").manual_seed(205)
    vals = torch.tensor([0.0, 0.5, -0.5, 1.0, -1.0])
    qI = synth.encode_e4m3(vals[torch.randint(5, (B, T, H, d_I), generator=g)])
    kI = synth.encode_e4m3(vals[torch.randint(5, (B, S, d_I), generator=g)])
    w = (torch.randint(-16, 17, (B, T, H), generator=g).float() / 64.0)
    pos0 = torch.tensor([S - T], dtype=torch.int32)
    kvl = torch.tensor([S], dtype=torch.int32)
    qa = torch.randn(B, T, H_q, d, generator=g).to(torch.bfloat16)
    Ka = (torch.randn(B, S, 1, d, generator=g) * 0.5).to(torch.bfloat16)
    Va = torch.randn(B, S, 1, d, generator=g).to(torch.bfloat16)

    # GPU chain
    dev = {n: v.to(DEV) for n, v in (("qI", qI), ("kI", kI), ("w", w), ("pos0", pos0),
                                     ("kvl", kvl), ("q", qa), ("K", Ka), ("V", Va))}
    idx, sel = bd.topk(dev["qI"], dev["kI"], dev["w"], dev["pos0"], dev["kvl"], k, with_scores=True)
    _, lse = bd.sparse_attention(dev["q"], dev["K"], dev["V"], idx, scale, kv_len=dev["kvl"],
                                 with_lse=True)
    sel_t = (sel * temp).contiguous()
    _, dsc = bd.indexer_kl(dev["q"], dev["K"], idx, lse, sel_t, scale, kv_len=dev["kvl"])
    args = bd.indexer_args(dev["qI"], dev["kI"], dev["w"], dev["pos0"], dev["kvl"])
    got = bd.indexer_bwd(args, idx, dsc, DEV)
    torch.cuda.synchronize()
    got = tuple(x.cpu().numpy() for x in got)

    # oracle chain on the host inputs
    qI_h, kI_h, w_h = qI.numpy(), kI.numpy(), w.numpy().astype(np.float64)
    rows = list(range(T))
    ref_idx, ref_sc = O.topk_rows(qI_h, kI_h, w_h, pos0.numpy(), kvl.numpy(), 0, rows, k,
                                  return_scores=True)
    assert np.array_equal(idx[0].cpu().numpy(), ref_idx), "selection differs"
    kept = np.full((T, k), -np.inf)
    for t in rows:
        v = ref_idx[t] >= 0
        kept[t, v] = ref_sc[t][ref_idx[t][v]]
    assert np.array_equal(sel[0].cpu().numpy().astype(np.float64)[np.isfinite(kept)],
                          kept[np.isfinite(kept)]), "kept scores differ"
    qb, Kb = synth.bf16_bits(qa), synth.bf16_bits(Ka)
    _, ref_ds = O.indexer_kl_rows(qb, Kb, ref_idx, kept * temp, 0, rows, scale, S)
    # the KL gradient's tolerance (as in the KL parity tests), carried through |.|
    qf, Kf = O.decode_bf16(qb)[0], O.decode_bf16(Kb)[0]
    eps = np.zeros((T, k))
    for t in rows:
        v = ref_idx[t] >= 0
        L = float(np.abs(scale * (Kf[ref_idx[t][v], 0, :] @ qf[t].T)).max())
        s = kept[t, v] * temp
        e = np.exp(s - s.max())
        pred = e / e.sum()
        eps[t, v] = 2e-5 * (1 + L) * np.maximum(pred, np.abs(pred - ref_ds[t, v])) + 1e-7
    prop = O.indexer_backward_rows(abs_codes(qI_h), abs_codes(kI_h), np.abs(w_h), ref_idx,
                                   eps, 0, rows, S)
    got_ds = dsc[0].cpu().numpy()
    assert np.all(np.abs(got_ds - ref_ds) <= eps), "dscores out of the KL tolerance"
    check_indexer_bwd(got, qI_h, kI_h, w_h, ref_idx[None].astype(np.int32), ref_ds[None], kvl.numpy(),
           extra=[prop])


def test_indexer_bwd_deterministic_dq_dw():
    """dq_I and dw are plain sums in a fixed order: bitwise equal from run to run.  dk_I is
    accumulated with float atomics, so only its value (not its last bits) is fixed."""
    say("[ix_indexer_bwd] determinism")
    qI, kI, w, kvl, idx, ds = _case(206, 1, 24, 700, 64, 128, 160, [700])
    a = _run(qI, kI, w, kvl, idx, ds)
    b = _run(qI, kI, w, kvl, idx, ds)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    scale = np.abs(a[2]).max()
    assert np.abs(a[2] - b[2]).max() <= 1e-5 * scale


def test_indexer_bwd_atomic_free_is_reproducible():
    """Without atomics each key lists its pairs in row order, so dk_I too is bitwise equal from
    run to run: one pass over many row blocks, and passes of 40 rows."""
    say("[ix_indexer_bwd] atomic-free determinism")
    qI, kI, w, kvl, idx, ds = _case(207, 2, 300, 700, 64, 128, 160, [700, 650])
    for rows_per_pass, pair_rows in ((1 << 20, BF), (40, BF), (40, F32)):
        a = _run(qI, kI, w, kvl, idx, ds, rows_per_pass=rows_per_pass, pair_rows=pair_rows)
        b = _run(qI, kI, w, kvl, idx, ds, rows_per_pass=rows_per_pass, pair_rows=pair_rows)
        for x, y, name in zip(a, b, ("dq_I", "dw", "dk_I")):
            assert np.array_equal(x, y), (f"{name} differs between runs ({rows_per_pass} rows per "
                                          f"pass, pair rows {pair_rows})")


def test_indexer_bwd_fp32_rows_match_atomics():
    """With fp32 dk_I pair rows the atomic-free form adds the same fp32 rows as the atomic
    form, only in another order: dk_I agrees with the atomics to fp32 reordering, far inside
    the bf16 rows' distance; dq_I and dw are the same computation (bitwise)."""
    say("[ix_indexer_bwd] fp32 pair rows vs atomics, keys kept by many rows")
    qI, kI, w, kvl, idx, ds = _case(208, 1, 200, 300, 64, 128, 128, [300])
    a = _run(qI, kI, w, kvl, idx, ds)
    f16 = _run(qI, kI, w, kvl, idx, ds, rows_per_pass=30, pair_rows=BF)
    f32 = _run(qI, kI, w, kvl, idx, ds, rows_per_pass=30, pair_rows=F32)
    for got in (f16, f32):
        assert np.array_equal(a[0], got[0]) and np.array_equal(a[1], got[1])
    mag = O.indexer_backward_rows(abs_codes(qI), abs_codes(kI), np.abs(w), idx[0], np.abs(ds[0]),
                                  0, list(range(200)), int(kvl[0]))[2]
    # two orders of the same fp32 additions: at most (T + 64) u of the magnitude each
    bound = 2 * (200 + 64) * 2.0 ** -24 * mag
    err32 = np.abs(f32[2][0].astype(np.float64) - a[2][0])
    assert np.all(err32 <= bound), f"fp32 rows off the atomics by up to {(err32 / np.maximum(bound, 1e-300)).max():.2f} bounds"
    dev16 = np.abs(f16[2] - a[2]).max()
    say(f"  max |bf16 rows - atomics| {dev16:.3e}, max |fp32 rows - atomics| {err32.max():.3e}")
    assert err32.max() * 16 <= dev16
