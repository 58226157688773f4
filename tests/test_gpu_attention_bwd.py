"""GPU parity: sparse-attention gradients (sparse_attn_bwd, indexshare_group_bwd) against the
oracle's chain rule, entry by entry.

Tolerance (parity_util.attn_bwd_bounds): each entry of dq, dK and dV is a sum of terms, and
every rounding the kernels make -- bf16 P and dS in the matrix products, D = dout . out from
the bf16 forward output, the atomic-free form's pair rows when they are bf16, MFMA and fp32
sums -- moves it
by at most a small multiple (a few 2^-8) of sums of magnitudes along the chain rule that the
oracle forms for that entry (O.sparse_attention_backward_magnitudes).  Each entry must lie
within that worst-case bound of the oracle; an entry that no query reaches has bound 0 and
must be exactly 0.  The checks also require that most nonzero entries exceed their own
bound, so a missing or misplaced key row could not pass.
"""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from oracle import ix_oracle as O
from parity_util import (BF16_MFMA_REL, BF16_U, FP32_U, attn_bwd_bounds, check_attn_bwd_entries,
                         logit_magnitude, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def check_backward(got, q_bits, K_bits, V_bits, idx, kvl, dout, scale, pair_rows, where,
                   power=0.6):
    """got = (dq, dK, dV) host arrays [B,T,H_q,d], [B,S,H_kv,d], [B,S,H_kv,d]; the oracle runs
    on every row of every sequence.  Returns the worst err / bound per gradient."""
    gq, gK, gV = got
    B, T, H_q, d = gq.shape
    k = idx.shape[2]
    worst = np.zeros(3)
    for b in range(B):
        ridx = np.where((idx[b] >= 0) & (idx[b] < kvl[b]), idx[b], -1)
        rows = list(range(T))
        do = dout[b].astype(np.float64)
        ref = O.sparse_attention_backward_rows(q_bits, K_bits, V_bits, ridx, do, b, rows, scale)
        mags = O.sparse_attention_backward_magnitudes(q_bits, K_bits, V_bits, ridx, do, b, rows,
                                                      scale)
        lm = logit_magnitude(O.decode_bf16(q_bits[b]), O.decode_bf16(K_bits[b]), scale)
        bounds = attn_bwd_bounds(mags, k, T, H_q, d, lm, pair_rows)
        for n, (g, r, bd_) in enumerate(zip((gq[b], gK[b], gV[b]), ref, bounds)):
            name = ("dq", "dK", "dV")[n]
            worst[n] = max(worst[n], check_attn_bwd_entries(g, r, bd_, f"{where} {name} b={b}",
                                                            power=power))
        for t in range(T):
            if (ridx[t] < 0).all():
                assert np.all(gq[b, t] == 0), f"{where}: empty row b={b} t={t}"
    say(f"  {where}: worst err / bound: dq {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}")
    return worst


def _pair_bounds(mags, n_rows, H_q, orders, pair_rows):
    """Bounds on the difference of two computations of dK and dV from the same dS and P that
    add in different orders (orders: 2 = both sums reorder) and, with pair_rows, one of them
    rounds each pair row to bf16."""
    g = BF16_MFMA_REL + (n_rows * H_q + 64) * FP32_U
    grow = 1.03  # computed |dS| and bf16 P over the exact magnitudes (f of attn_bwd_bounds, with room)
    c = (BF16_U * (1 + g) if pair_rows else 0.0) + orders * (n_rows * H_q + 64) * FP32_U
    mk = mags["dK"]
    sk = grow * (mk["ds"] + BF16_MFMA_REL * mk["dp"] + 0.02 * mk["dd"])
    return c * sk, c * grow * mags["dV"]["p"]


def _form(rows_per_pass, pair_rows):
    if rows_per_pass is None:
        return "atomics"
    rows = "fp32" if pair_rows == bd.PAIR_ROWS_FP32 else "bf16"
    return f"key-major, {rows_per_pass} rows per pass, {rows} pair rows"


def _run(B, T, S, H_q, H_kv, d, k, seed, kv_lens=None, empty_rows=(), rows_per_pass=None,
         pair_rows=bd.PAIR_ROWS_BF16):
    say(f"[sparse_attn_bwd] B={B} T={T} S={S} H_q={H_q} H_kv={H_kv} d={d} k={k} seed={seed} "
        f"{_form(rows_per_pass, pair_rows)}")
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = (torch.randn(B, T, H_q, d, generator=g) * 0.3).to(torch.bfloat16)
    K = (torch.randn(B, S, H_kv, d, generator=g) * 0.3).to(torch.bfloat16)
    V = torch.randn(B, S, H_kv, d, generator=g).to(torch.bfloat16)
    dout = torch.randn(B, T, H_q, d, generator=g).to(torch.bfloat16)
    kvl = np.array(kv_lens if kv_lens is not None else [S] * B, dtype=np.int32)
    rng = np.random.default_rng(seed)
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            if (b, t) in empty_rows:
                continue
            n = int(rng.integers(1, k + 1))
            sel = np.sort(rng.choice(S, size=n, replace=False))   # may include >= kv_len: skipped
            idx[b, t, :n] = sel
    dq_, dK_, dV_ = (x.to(DEV) for x in (q, K, V))
    didx = torch.from_numpy(idx).to(DEV)
    dkvl = torch.from_numpy(kvl).to(DEV)
    scale = d ** -0.5
    out, lse = bd.sparse_attention(dq_, dK_, dV_, didx, scale, kv_len=dkvl, with_lse=True)
    gq, gK, gV = bd.sparse_attention_backward(dq_, dK_, dV_, didx, out, lse, dout.to(DEV), scale,
                                              kv_len=dkvl, rows_per_pass=rows_per_pass,
                                              pair_rows=pair_rows)
    torch.cuda.synchronize()
    got = (gq.cpu().numpy(), gK.cpu().numpy(), gV.cpu().numpy())
    check_backward(got, _bits(q), _bits(K), _bits(V), idx, kvl, dout.float().numpy(), scale,
                   rows_per_pass is not None and pair_rows == bd.PAIR_ROWS_BF16, "sparse_attn_bwd")


# (rows_per_pass, pair_rows).  None: dK / dV added with atomics; a row count: the atomic-free
# form (inverted selection, per-pair rows, key-major sums), in passes of that many query rows,
# with bf16 or fp32 pair rows
MODES = [(None, bd.PAIR_ROWS_BF16), (1 << 20, bd.PAIR_ROWS_BF16), (7, bd.PAIR_ROWS_BF16),
         (1 << 20, bd.PAIR_ROWS_FP32), (7, bd.PAIR_ROWS_FP32)]


@pytest.mark.parametrize("rows_per_pass,pair_rows", MODES)
def test_backward_gqa_ragged_d64(rows_per_pass, pair_rows):
    _run(B=2, T=40, S=300, H_q=8, H_kv=2, d=64, k=48, seed=71, kv_lens=[300, 170],
         empty_rows={(0, 3)}, rows_per_pass=rows_per_pass, pair_rows=pair_rows)


@pytest.mark.parametrize("rows_per_pass,pair_rows", MODES)
def test_backward_mqa_d128_many_chunks(rows_per_pass, pair_rows):
    _run(B=1, T=64, S=4096, H_q=16, H_kv=1, d=128, k=256, seed=72, rows_per_pass=rows_per_pass,
         pair_rows=pair_rows)


@pytest.mark.parametrize("rows_per_pass,pair_rows", MODES)
def test_backward_k_not_a_multiple_of_4(rows_per_pass, pair_rows):
    _run(B=1, T=33, S=500, H_q=16, H_kv=1, d=128, k=37, seed=73, rows_per_pass=rows_per_pass,
         pair_rows=pair_rows)


def test_backward_atomic_free_matches_atomics():
    """The forms sum the same fp32 products; the atomic-free one with bf16 pair rows rounds
    each pair's rows to bf16 first, so dK and dV agree to bf16 rounding of the terms; with fp32
    pair rows only the order of the fp32 sums differs.  dq is the same computation (bitwise)."""
    say("[sparse_attn_bwd] atomic-free vs atomics, hot keys shared by every query")
    g = torch.Generator(device="cpu").manual_seed(74)
    B, T, S, H_q, d, k = 2, 48, 600, 16, 128, 64
    q = (torch.randn(B, T, H_q, d, generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    K = (torch.randn(B, S, 1, d, generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    V = torch.randn(B, S, 1, d, generator=g).to(torch.bfloat16).to(DEV)
    dout = torch.randn(B, T, H_q, d, generator=g).to(torch.bfloat16).to(DEV)
    rng = np.random.default_rng(74)
    idx = np.stack([np.stack([np.sort(np.concatenate([np.arange(16), 16 + rng.choice(S - 16, k - 16,
                                                                                  replace=False)]))
                              for _ in range(T)]) for _ in range(B)]).astype(np.int32)
    didx = torch.from_numpy(idx).to(DEV)
    out, lse = bd.sparse_attention(q, K, V, didx, d ** -0.5, with_lse=True)
    a = bd.sparse_attention_backward(q, K, V, didx, out, lse, dout, d ** -0.5)
    f = bd.sparse_attention_backward(q, K, V, didx, out, lse, dout, d ** -0.5, rows_per_pass=10)
    f32 = bd.sparse_attention_backward(q, K, V, didx, out, lse, dout, d ** -0.5, rows_per_pass=10,
                                       pair_rows=bd.PAIR_ROWS_FP32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], f[0]) and torch.equal(a[0], f32[0]), "dq differs"
    # per entry: the bf16 atomic-free form's only extra rounding is each pair row's bf16
    # rounding; the fp32 one has none; and the forms add in different orders
    qb, Kb, Vb = _bits(q), _bits(K), _bits(V)
    dob = dout.float().cpu().numpy().astype(np.float64)
    for b in range(B):
        mags = O.sparse_attention_backward_magnitudes(qb, Kb, Vb, idx[b], dob[b], b,
                                                      list(range(T)), d ** -0.5)
        for got, bf16_rows, form in ((f, True, "bf16 rows"), (f32, False, "fp32 rows")):
            bK, bV = _pair_bounds(mags, T, H_q, 2, bf16_rows)
            for n, bnd in ((1, bK), (2, bV)):
                x = a[n][b].double().cpu().numpy()
                y = got[n][b].double().cpu().numpy()
                # the fp32 rows differ from the atomics only by reordering: few entries come
                # near that bound, so no share of them is asked to
                check_attn_bwd_entries(y, x, bnd, f"{('dK', 'dV')[n - 1]} b={b}: atomic-free "
                                       f"({form}) vs atomics", power=0.5 if bf16_rows else None)
    # fp32 rows sit far closer to the atomic form than bf16 rows do
    for n in (1, 2):
        dev16 = (f[n] - a[n]).abs().max().item()
        dev32 = (f32[n] - a[n]).abs().max().item()
        say(f"  {('dK', 'dV')[n - 1]}: max |bf16 rows - atomics| {dev16:.3e}, "
            f"max |fp32 rows - atomics| {dev32:.3e}")
        assert dev32 * 16 <= dev16, "fp32 pair rows are not tighter than bf16 ones"
    # and every form against the oracle
    for form, got in (("atomics", a), ("atomic-free", f), ("atomic-free fp32 rows", f32)):
        # 16 hot keys kept by every query sum 768 terms each, so fewer entries stand out
        check_backward(tuple(x.cpu().numpy() for x in got), qb, Kb, Vb, idx, np.array([S] * B),
                       dout.float().cpu().numpy(), d ** -0.5, form == "atomic-free", form,
                       power=0.5)


def test_atomic_free_backward_is_reproducible():
    """Without atomics each key lists its pairs in row order, so dK and dV are bitwise equal
    from run to run: one pass over many row blocks, and passes of 50 rows.  Keys drawn from a
    short range are kept by many rows, so their segments span many row blocks."""
    say("[sparse_attn_bwd] atomic-free determinism")
    g = torch.Generator(device="cpu").manual_seed(91)
    B, T, S, H_q, H_kv, d, k = 2, 400, 900, 16, 1, 128, 192
    q = (torch.randn(B, T, H_q, d, generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    K = (torch.randn(B, S, H_kv, d, generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    V = torch.randn(B, S, H_kv, d, generator=g).to(torch.bfloat16).to(DEV)
    dout = torch.randn(B, T, H_q, d, generator=g).to(torch.bfloat16).to(DEV)
    rng = np.random.default_rng(91)
    idx = np.stack([np.stack([np.sort(rng.choice(S // 3, size=k, replace=False)) for _ in range(T)])
                    for _ in range(B)]).astype(np.int32)
    didx = torch.from_numpy(idx).to(DEV)
    scale = d ** -0.5
    out, lse = bd.sparse_attention(q, K, V, didx, scale, with_lse=True)
    for rows_per_pass, pair_rows in ((1 << 20, bd.PAIR_ROWS_BF16), (50, bd.PAIR_ROWS_BF16),
                                     (50, bd.PAIR_ROWS_FP32)):
        runs = [bd.sparse_attention_backward(q, K, V, didx, out, lse, dout, scale,
                                             rows_per_pass=rows_per_pass, pair_rows=pair_rows)
                for _ in range(2)]
        torch.cuda.synchronize()
        for x, y, name in zip(runs[0], runs[1], ("dq", "dK", "dV")):
            assert torch.equal(x, y), f"{name} differs between runs ({_form(rows_per_pass, pair_rows)})"


@pytest.mark.parametrize("rows_per_pass,pair_rows", [(None, bd.PAIR_ROWS_BF16),
                                                    (10, bd.PAIR_ROWS_BF16),
                                                    (10, bd.PAIR_ROWS_FP32)])
def test_group_backward_shares_the_inversion(rows_per_pass, pair_rows):
    """indexshare_group_bwd: three layers over one selection, the selection inverted once per
    pass.  Each layer equals sparse_attn_bwd's atomic-free form on its own inputs (dq bit for
    bit; dK, dV up to the order of the per-key fp32 sums), and the oracle's chain rule."""
    say(f"[indexshare_group_bwd] 3 layers, {_form(rows_per_pass or 'all', pair_rows)}")
    g = torch.Generator(device="cpu").manual_seed(75)
    B, T, S, H_q, H_kv, d, k = 2, 30, 400, 8, 2, 64, 40
    rng = np.random.default_rng(75)
    kvl = np.array([400, 260], dtype=np.int32)
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            n = int(rng.integers(1, k + 1))
            idx[b, t, :n] = np.sort(rng.choice(S, size=n, replace=False))
    didx = torch.from_numpy(idx).to(DEV)
    dkvl = torch.from_numpy(kvl).to(DEV)
    scale = d ** -0.5
    layers = []
    for _ in range(3):
        q = (torch.randn(B, T, H_q, d, generator=g) * 0.3).to(torch.bfloat16)
        K = (torch.randn(B, S, H_kv, d, generator=g) * 0.3).to(torch.bfloat16)
        V = torch.randn(B, S, H_kv, d, generator=g).to(torch.bfloat16)
        dout = torch.randn(B, T, H_q, d, generator=g).to(torch.bfloat16)
        L = {n: x.to(DEV) for n, x in (("q", q), ("K", K), ("V", V), ("dout", dout))}
        L["out"], L["lse"] = bd.sparse_attention(L["q"], L["K"], L["V"], didx, scale, kv_len=dkvl,
                                                 with_lse=True)
        layers.append(L)
    grads = bd.group_attention_backward(didx, layers, scale, kv_len=dkvl, rows_per_pass=rows_per_pass,
                                        pair_rows=pair_rows)
    torch.cuda.synchronize()
    for l, L in enumerate(layers):
        ref = bd.sparse_attention_backward(L["q"], L["K"], L["V"], didx, L["out"], L["lse"], L["dout"],
                                           scale, kv_len=dkvl, rows_per_pass=rows_per_pass or B * T,
                                           pair_rows=pair_rows)
        torch.cuda.synchronize()
        assert torch.equal(grads[l][0], ref[0]), f"layer {l}: dq differs"
        # the same pair rows, summed per key in fp32 (in row order in both)
        qb, Kb, Vb = _bits(L["q"]), _bits(L["K"]), _bits(L["V"])
        dob = L["dout"].float().cpu().numpy().astype(np.float64)
        for b in range(B):
            ridx = np.where((idx[b] >= 0) & (idx[b] < kvl[b]), idx[b], -1)
            mags = O.sparse_attention_backward_magnitudes(qb, Kb, Vb, ridx, dob[b], b,
                                                          list(range(T)), scale)
            bK, bV = _pair_bounds(mags, T, H_q, 2, False)
            for n, bnd in ((1, bK), (2, bV)):
                check_attn_bwd_entries(grads[l][n][b].double().cpu().numpy(),
                                       ref[n][b].double().cpu().numpy(), bnd,
                                       f"layer {l} {('dK', 'dV')[n - 1]} b={b}: group vs single")
    # and every layer against the oracle
    for l, L in enumerate(layers):
        check_backward(tuple(x.cpu().numpy() for x in grads[l]), _bits(L["q"]), _bits(L["K"]),
                       _bits(L["V"]), idx, kvl, L["dout"].float().cpu().numpy(), scale,
                       pair_rows == bd.PAIR_ROWS_BF16, f"group layer {l}")
