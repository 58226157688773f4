"""GPU parity: sparse-attention gradients (sparse_attn_bwd) against the oracle's chain rule.

Tolerance.  The kernel rounds P and dS to bf16 for the matrix products (relative 2^-9
each) and takes D = dout . out from the bf16-rounded forward output; everything else is
fp32 accumulation of exact bf16 products.  A gradient is a sum of such terms, so it is
checked in norm: per query (dq) and per sequence (dK, dV), ||g - g_ref|| <= 2e-2 ||g_ref||
plus an absolute floor of 1e-4 sqrt(n) times the size of one term,
sm_scale max|K| max|dout| max|V| (an exact zero, e.g. dq of a query with one valid key,
comes back as bf16 rounding noise).
"""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from oracle import ix_oracle as O
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL = 2e-2


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _close(g, ref, term, what):
    scale = np.linalg.norm(ref)
    err = np.linalg.norm(g - ref)
    assert err <= REL * scale + 1e-4 * term * np.sqrt(ref.size), \
        f"{what}: |err| {err:.3e} vs |ref| {scale:.3e}"


def _run(B, T, S, H_q, H_kv, d, k, seed, kv_lens=None, empty_rows=(), rows_per_pass=None):
    say(f"[sparse_attn_bwd] B={B} T={T} S={S} H_q={H_q} H_kv={H_kv} d={d} k={k} seed={seed} "
        f"{'atomics' if rows_per_pass is None else f'key-major, {rows_per_pass} rows per pass'}")
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
                                              kv_len=dkvl, rows_per_pass=rows_per_pass)
    torch.cuda.synchronize()
    gq, gK, gV = gq.cpu().numpy(), gK.cpu().numpy(), gV.cpu().numpy()
    term = scale * float(K.float().abs().max() * dout.float().abs().max() * V.float().abs().max())
    for b in range(B):
        ridx = np.where((idx[b] >= 0) & (idx[b] < kvl[b]), idx[b], -1)
        rq, rK, rV = O.sparse_attention_backward_rows(
            _bits(q), _bits(K), _bits(V), ridx, dout[b].float().numpy().astype(np.float64), b,
            list(range(T)), scale)
        for t in range(T):
            if (ridx[t] < 0).all():
                assert np.all(gq[b, t] == 0), f"empty row b={b} t={t}"
            else:
                _close(gq[b, t], rq[t], term, f"dq b={b} t={t}")
        _close(gK[b], rK, term, f"dK b={b}")
        _close(gV[b], rV, term, f"dV b={b}")
        untouched = np.setdiff1d(np.arange(S), ridx[ridx >= 0])
        assert np.all(gK[b, untouched] == 0) and np.all(gV[b, untouched] == 0)


# None: dK / dV added with atomics; a row count: the atomic-free form (inverted selection,
# per-pair rows, key-major sums), in passes of that many query rows
MODES = [None, 1 << 20, 7]


@pytest.mark.parametrize("rows_per_pass", MODES)
def test_backward_gqa_ragged_d64(rows_per_pass):
    _run(B=2, T=40, S=300, H_q=8, H_kv=2, d=64, k=48, seed=71, kv_lens=[300, 170],
         empty_rows={(0, 3)}, rows_per_pass=rows_per_pass)


@pytest.mark.parametrize("rows_per_pass", MODES)
def test_backward_mqa_d128_many_chunks(rows_per_pass):
    _run(B=1, T=64, S=4096, H_q=16, H_kv=1, d=128, k=256, seed=72, rows_per_pass=rows_per_pass)


@pytest.mark.parametrize("rows_per_pass", MODES)
def test_backward_k_not_a_multiple_of_4(rows_per_pass):
    _run(B=1, T=33, S=500, H_q=16, H_kv=1, d=128, k=37, seed=73, rows_per_pass=rows_per_pass)


def test_backward_atomic_free_matches_atomics():
    """The two forms sum the same fp32 products; the atomic-free one rounds each pair's rows
    to bf16 first, so dK and dV agree to bf16 rounding of the terms, and dq is the same
    computation (bitwise)."""
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
    torch.cuda.synchronize()
    assert torch.equal(a[0], f[0]), "dq differs"
    for n, (x, y) in enumerate(zip(a[1:], f[1:])):
        err = float((x - y).norm())
        assert err <= 4e-3 * float(x.norm()), f"{('dK', 'dV')[n]}: {err:.3e} vs {float(x.norm()):.3e}"


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
    for rows_per_pass in (1 << 20, 50):
        runs = [bd.sparse_attention_backward(q, K, V, didx, out, lse, dout, scale,
                                             rows_per_pass=rows_per_pass) for _ in range(2)]
        torch.cuda.synchronize()
        for x, y, name in zip(runs[0], runs[1], ("dq", "dK", "dV")):
            assert torch.equal(x, y), f"{name} differs between runs ({rows_per_pass} rows per pass)"


@pytest.mark.parametrize("rows_per_pass", [None, 10])
def test_group_backward_shares_the_inversion(rows_per_pass):
    """indexshare_group_bwd: three layers over one selection, the selection inverted once per
    pass.  Each layer equals sparse_attn_bwd's atomic-free form on its own inputs (dq bit for
    bit; dK, dV up to the order of the per-key fp32 sums), and the oracle's chain rule."""
    say(f"[indexshare_group_bwd] 3 layers, rows per pass {rows_per_pass}")
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
    grads = bd.group_attention_backward(didx, layers, scale, kv_len=dkvl, rows_per_pass=rows_per_pass)
    torch.cuda.synchronize()
    for l, L in enumerate(layers):
        ref = bd.sparse_attention_backward(L["q"], L["K"], L["V"], didx, L["out"], L["lse"], L["dout"],
                                           scale, kv_len=dkvl, rows_per_pass=rows_per_pass or B * T)
        torch.cuda.synchronize()
        assert torch.equal(grads[l][0], ref[0]), f"layer {l}: dq differs"
        for n in (1, 2):
            err = float((grads[l][n].double() - ref[n].double()).norm())
            assert err <= 1e-5 * float(ref[n].double().norm()), f"layer {l}: {('dK', 'dV')[n - 1]}"
    # and layer 1 against the oracle
    L = layers[1]
    gq, gK, gV = (x.cpu().numpy() for x in grads[1])
    term = scale * float(L["K"].float().abs().max() * L["dout"].float().abs().max() *
                         L["V"].float().abs().max())
    for b in range(B):
        ridx = np.where((idx[b] >= 0) & (idx[b] < kvl[b]), idx[b], -1)
        rq, rK, rV = O.sparse_attention_backward_rows(
            _bits(L["q"]), _bits(L["K"]), _bits(L["V"]), ridx,
            L["dout"][b].float().cpu().numpy().astype(np.float64), b, list(range(T)), scale)
        for t in range(T):
            _close(gq[b, t], rq[t], term, f"dq b={b} t={t}")
        _close(gK[b], rK, term, f"dK b={b}")
        _close(gV[b], rV, term, f"dV b={b}")
