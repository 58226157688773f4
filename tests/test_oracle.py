"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: exact integer arithmetic,
rational brute force, torch library routines (fp8/bf16 casts, SDPA), closed forms and
inputs built so that the answer is known by construction.
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ix_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- storage formats


def test_e4m3_table_matches_torch_and_spec_points():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.decode_e4m3(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # spec points of OCP E4M3
    assert ours[0x00] == 0.0 and ours[0x80] == 0.0 and math.copysign(1, ours[0x80]) == -1
    assert ours[0x01] == 2.0 ** -9          # smallest subnormal
    assert ours[0x08] == 2.0 ** -6          # smallest normal
    assert ours[0x38] == 1.0
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0


def test_e4m3_values_are_multiples_of_2pow_minus9():
    v = O.decode_e4m3(np.arange(256, dtype=np.uint8))
    v = v[~np.isnan(v)]
    scaled = v * 512.0
    assert np.array_equal(scaled, np.round(scaled))
    assert np.abs(v).max() < 2 ** 9


def _nearest_e4m3_brute_force(v):
    """Nearest finite e4m3 code to clamp(v, -448, 448) by scanning all 256 codes; ties go
    to the code with an even mantissa (even code), zero keeps the sign of v."""
    a = max(-448.0, min(448.0, v))
    best, best_d = None, None
    for c in range(256):
        x = O.E4M3_TABLE[c]
        if math.isnan(x) or (x == 0 and (c & 0x80) != (0x80 if math.copysign(1, v) < 0 else 0)):
            continue
        if x != 0 and (x < 0) != (a < 0):
            continue
        d = abs(Fraction(x) - Fraction(a))
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def test_encode_e4m3_round_trips_every_code():
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    back = O.encode_e4m3(O.E4M3_TABLE[codes])
    assert back.tolist() == codes


def test_encode_e4m3_matches_brute_force_nearest():
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(300) * 4.0) + list(rng.standard_normal(200) * 2.0 ** -7)
    vals += list(rng.uniform(-500, 500, 100))
    # every midpoint between neighbouring finite magnitudes, and just either side of it
    mags = sorted(set(abs(x) for x in O.E4M3_TABLE if not math.isnan(x)))
    for lo, hi in zip(mags, mags[1:]):
        m = (lo + hi) / 2
        vals += [m, -m, np.nextafter(m, 0.0), np.nextafter(m, 1e9)]
    vals = [float(np.float32(v)) for v in vals]
    got = O.encode_e4m3(np.array(vals))
    want = [_nearest_e4m3_brute_force(v) for v in vals]
    assert got.tolist() == want


def test_encode_e4m3_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.standard_normal(4000) * 3, rng.standard_normal(1000) * 1e-2,
                        rng.uniform(-1000, 1000, 1000)]).astype(np.float32)
    ref = torch.from_numpy(x).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_e4m3(x), ref)


def test_encode_e4m3_specials():
    enc = lambda v: int(O.encode_e4m3(np.array([v]))[0])  # noqa: E731
    assert enc(1e30) == 0x7E and enc(-1e30) == 0xFE and enc(464.0) == 0x7E   # saturate
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -10) == 0x00 and enc(-(2.0 ** -10)) == 0x80             # tie to 0
    assert enc(3 * 2.0 ** -10) == 0x02                                          # tie to even
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A                          # ties to even
    assert enc(float("nan")) in (0x7F, 0xFF)


def test_append_kv_writes_only_target_rows():
    rng = np.random.default_rng(7)
    B, S, T_new, d_I, H, d = 3, 10, 2, 8, 2, 4
    kc = rng.integers(0, 256, (B, S, d_I), dtype=np.uint8)
    Kc = rng.integers(0, 1 << 16, (B, S, H, d), dtype=np.uint16)
    Vc = rng.integers(0, 1 << 16, (B, S, H, d), dtype=np.uint16)
    kn = rng.standard_normal((B, T_new, d_I)).astype(np.float32)
    Kn = rng.integers(0, 1 << 16, (B, T_new, H, d), dtype=np.uint16)
    Vn = rng.integers(0, 1 << 16, (B, T_new, H, d), dtype=np.uint16)
    pos0 = np.array([3, 9, -1])   # sequence 1's second token and sequence 2's first fall outside
    k2, K2, V2 = O.append_kv(kc, Kc, Vc, kn, Kn, Vn, pos0)
    written = {(0, 3): (0, 0), (0, 4): (0, 1), (1, 9): (1, 0), (2, 0): (2, 1)}
    for b in range(B):
        for s in range(S):
            if (b, s) in written:
                bb, t = written[(b, s)]
                assert np.array_equal(k2[b, s], O.encode_e4m3(kn[bb, t]))
                assert np.array_equal(K2[b, s], Kn[bb, t]) and np.array_equal(V2[b, s], Vn[bb, t])
            else:
                assert np.array_equal(k2[b, s], kc[b, s])
                assert np.array_equal(K2[b, s], Kc[b, s]) and np.array_equal(V2[b, s], Vc[b, s])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = O.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ---------------------------------------------------------------- stage 1: scores


def _rand_codes(rng, shape, finite=True):
    c = rng.integers(0, 256, size=shape, dtype=np.uint32).astype(np.uint8)
    if finite:
        c[(c & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    return c


def test_per_head_dot_is_exact_against_int64():
    rng = np.random.default_rng(1)
    for d in (64, 128):
        q = _rand_codes(rng, (64, d))
        k = _rand_codes(rng, (300, d))
        q[0, :] = 0x7E   # +448 everywhere: the largest magnitude case
        k[0, :] = 0x7E
        k[1, :] = 0xFE   # -448
        qi = (O.decode_e4m3(q) * 512).astype(np.int64)
        ki = (O.decode_e4m3(k) * 512).astype(np.int64)
        exact = qi @ ki.T                          # integers, exact in int64
        x = O.decode_e4m3(q) @ O.decode_e4m3(k).T  # what index_scores forms
        assert np.array_equal(x * 2.0 ** 18, exact.astype(np.float64))
        assert np.array_equal((x * 2.0 ** 18).astype(np.int64), exact)


def _fraction_scores(q_codes, k_codes, w, n):
    """Brute force: sum_h w_h * max(0, sum_c q*k) in exact rationals."""
    H, d = q_codes.shape
    qv = [[Fraction(float(O.E4M3_TABLE[q_codes[h, c]])) for c in range(d)] for h in range(H)]
    out = []
    for s in range(n):
        kv = [Fraction(float(O.E4M3_TABLE[k_codes[s, c]])) for c in range(d)]
        tot = Fraction(0)
        for h in range(H):
            x = sum(qv[h][c] * kv[c] for c in range(d))
            tot += Fraction(float(w[h])) * max(Fraction(0), x)
        out.append(tot)
    return out


def test_scores_against_rational_brute_force():
    rng = np.random.default_rng(2)
    T, S, H, d = 7, 11, 3, 8
    q = _rand_codes(rng, (1, T, H, d))
    k = _rand_codes(rng, (1, S, d))
    w = rng.random((1, T, H)).astype(np.float32)
    pos0, kvl = np.array([2]), np.array([9])   # ragged: kv_len < S, queries start at 2
    got = O.score_matrix(q, k, w, pos0, kvl, 0, list(range(T)), S)
    for t in range(T):
        n = O.visible_count(2, 9, t)
        assert n == min(2 + t + 1, 9)
        ex = _fraction_scores(q[0, t], k[0], w[0, t], n)
        for s in range(S):
            if s < n:
                assert got[t, s] == pytest.approx(float(ex[s]), rel=1e-14, abs=1e-300)
            else:
                assert got[t, s] == -np.inf


def test_score_special_cases():
    rng = np.random.default_rng(3)
    q = _rand_codes(rng, (20, 1, 64))
    k = _rand_codes(rng, (50, 64))
    keys = O.decode_e4m3(k)
    # one head, weight 1: plain ReLU of the dot product
    for t in range(20):
        got = O.index_scores(O.decode_e4m3(q[t]), keys, np.ones(1))
        want = np.maximum(O.decode_e4m3(q[t, 0]) @ keys.T, 0)
        assert np.array_equal(got, want)
    # zero weights -> zero scores; doubling weights doubles scores exactly
    qh = O.decode_e4m3(_rand_codes(rng, (8, 64)))
    w = rng.random(8)
    assert np.all(O.index_scores(qh, keys, np.zeros(8)) == 0)
    assert np.array_equal(O.index_scores(qh, keys, 2 * w), 2 * O.index_scores(qh, keys, w))
    # permuting heads (queries and weights together) leaves scores unchanged
    perm = rng.permutation(8)
    a = O.index_scores(qh, keys, w)
    b = O.index_scores(qh[perm], keys, w[perm])
    assert np.allclose(a, b, rtol=1e-15, atol=0)
    # scores are >= 0 and are 0 exactly when every head's dot is <= 0
    x = qh @ keys.T
    assert np.all(a >= 0)
    assert np.array_equal(a == 0, np.all(x <= 0, axis=0))


# ---------------------------------------------------------------- stage 2: selection


def test_select_against_python_sort_with_ties():
    rng = random.Random(4)
    for trial in range(200):
        n = rng.randint(1, 40)
        k = rng.randint(1, 45)
        sc = np.array([rng.choice([0.0, 0.0, 1.5, 2.25, rng.random()]) for _ in range(n)])
        want = sorted(sorted(range(n), key=lambda s: (-sc[s], s))[: min(k, n)])
        got = O.select_topk(sc, k)
        assert got[: len(want)].tolist() == want
        assert np.all(got[len(want):] == -1)


def test_select_invariants():
    rng = np.random.default_rng(6)
    for n, k in [(1, 1), (5, 8), (100, 17), (64, 64), (1000, 1)]:
        sc = rng.random(n)
        sc[rng.integers(0, n, size=n // 3)] = 0.0
        got = O.select_topk(sc, k)
        sel = got[got >= 0]
        assert sel.size == min(k, n)
        assert np.all(np.diff(sel) > 0)              # ascending, distinct
        assert sel.min() >= 0 and sel.max() < n
        if k >= n:
            assert np.array_equal(sel, np.arange(n))  # everything visible is kept


def _e4m3_code(v):
    codes = np.nonzero(O.E4M3_TABLE == v)[0]
    assert codes.size >= 1
    return int(codes[0])


def test_sign_partitioned_planting_has_known_top_set():
    """Queries >= 0, unplanted keys <= 0: their scores are exactly 0.

    Planted keys have all coordinates equal to a distinct positive e4m3 value v_j, the
    query has all coordinates u, w = 1: score_j = H * d * u * v_j (closed form).
    The kept set is the planted keys, then the lowest-index zero-score keys.
    """
    rng = np.random.default_rng(7)
    S, H, d, k = 300, 4, 64, 40
    neg = [c for c in range(256) if O.E4M3_TABLE[c] <= 0 and not np.isnan(O.E4M3_TABLE[c])]
    k_codes = rng.choice(neg, size=(1, S, d)).astype(np.uint8)
    planted = sorted(rng.choice(np.arange(50, S), size=12, replace=False).tolist())
    vals = [0.5 + 0.0625 * i for i in range(8)] + [1.0 + 0.125 * i for i in range(4)]  # exact e4m3
    rng.shuffle(vals)
    for s, v in zip(planted, vals):
        k_codes[0, s, :] = _e4m3_code(v)
    u = 0.25
    q_codes = np.full((1, 1, H, d), _e4m3_code(u), dtype=np.uint8)
    w = np.ones((1, 1, H), dtype=np.float32)
    pos0, kvl = np.array([S - 1]), np.array([S])
    idx, scores = O.topk_rows(q_codes, k_codes, w, pos0, kvl, 0, [0], k, return_scores=True)
    sc = scores[0]
    for s, v in zip(planted, vals):
        assert sc[s] == H * d * u * v
    others = [s for s in range(S) if s not in planted]
    assert np.all(sc[others] == 0.0)
    want = sorted(planted + others[: k - len(planted)])
    assert idx[0].tolist() == want
    # with k below the planted count, only the best planted keys survive
    idx2 = O.topk_rows(q_codes, k_codes, w, pos0, kvl, 0, [0], 5)
    best = [s for s, _ in sorted(zip(planted, vals), key=lambda p: -p[1])[:5]]
    assert idx2[0].tolist() == sorted(best)


def test_query_sees_its_own_key_and_not_the_next():
    """Self-inclusion: only key p scores > 0 for the query at position p."""
    S, H, d = 16, 1, 64
    one = _e4m3_code(1.0)
    for p in range(S):
        k_codes = np.zeros((1, S, d), dtype=np.uint8)
        k_codes[0, p, :] = one
        if p + 1 < S:
            k_codes[0, p + 1, :] = _e4m3_code(2.0)   # future key, must stay invisible
        q_codes = np.full((1, 1, H, d), one, dtype=np.uint8)
        idx = O.topk_rows(q_codes, k_codes, np.ones((1, 1, H), np.float32),
                          np.array([p]), np.array([S]), 0, [0], 1)
        assert idx[0].tolist() == [p]


def test_golden_selection_constants():
    g = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    e = g["selection_limit_example"]
    rng = np.random.default_rng(8)
    sc = rng.random(e["previous_tokens"])
    got = O.select_topk(sc, e["limit"])
    assert (got >= 0).sum() == e["attended"]
    s = g["selection_size_at_1m"]
    assert round(100.0 * s["k"] / s["context"], 1) == s["percent_of_context_stated"]


# ---------------------------------------------------------------- attention


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _attn_case(rng, T=40, S=40, H_q=4, H_kv=2, d=16, scale_q=1.0):
    q = _bf16_bits(rng.standard_normal((1, T, H_q, d)) * scale_q)
    K = _bf16_bits(rng.standard_normal((1, S, H_kv, d)))
    V = _bf16_bits(rng.standard_normal((1, S, H_kv, d)))
    return q, K, V


def test_full_selection_equals_dense_causal_sdpa():
    rng = np.random.default_rng(9)
    T = S = 40
    H_q, H_kv, d = 4, 2, 16
    q, K, V = _attn_case(rng, T, S, H_q, H_kv, d)
    idx = np.array([[s if s <= t else -1 for s in range(S)] for t in range(T)])
    sm = 1.0 / math.sqrt(d)
    out, lse = O.sparse_attention_rows(q, K, V, idx, 0, list(range(T)), sm)
    qt = torch.from_numpy(O.decode_bf16(q[0])).permute(1, 0, 2)           # [H_q, T, d]
    Kt = torch.from_numpy(O.decode_bf16(K[0])).permute(1, 0, 2).repeat_interleave(H_q // H_kv, 0)
    Vt = torch.from_numpy(O.decode_bf16(V[0])).permute(1, 0, 2).repeat_interleave(H_q // H_kv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True, scale=sm)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    logits = (qt @ Kt.transpose(1, 2)) * sm
    mask = torch.ones(T, S, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)  # [H_q, T]
    assert np.allclose(lse, ref_lse.T.numpy(), rtol=1e-12, atol=1e-12)


def test_window_selection_equals_banded_sdpa():
    rng = np.random.default_rng(10)
    T = S = 48
    W, H_q, H_kv, d = 5, 2, 1, 32
    q, K, V = _attn_case(rng, T, S, H_q, H_kv, d)
    idx = np.full((T, 8), -1)
    for t in range(T):
        win = list(range(max(0, t - W + 1), t + 1))
        idx[t, : len(win)] = win
    sm = 0.3
    out, _ = O.sparse_attention_rows(q, K, V, idx, 0, list(range(T)), sm)
    qt = torch.from_numpy(O.decode_bf16(q[0])).permute(1, 0, 2)
    Kt = torch.from_numpy(O.decode_bf16(K[0])).permute(1, 0, 2).expand(H_q, S, d)
    Vt = torch.from_numpy(O.decode_bf16(V[0])).permute(1, 0, 2).expand(H_q, S, d)
    tt = torch.arange(T)[:, None]
    ss = torch.arange(S)[None, :]
    band = (ss <= tt) & (ss > tt - W)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=band, scale=sm)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(11)
    T, S, H_q, H_kv, d = 6, 30, 4, 1, 16
    q, K, V = _attn_case(rng, T, S, H_q, H_kv, d)
    Kf, Vf = O.decode_bf16(K[0]), O.decode_bf16(V[0])
    # k = 1: the output is the selected V row exactly, lse the single logit
    for t in range(T):
        j = int(rng.integers(0, S))
        out, lse = O.sparse_attention_row(O.decode_bf16(q[0, t]), Kf, Vf, np.array([j]), 0.7)
        for h in range(H_q):
            assert np.array_equal(out[h], Vf[j, 0])
            assert lse[h] == pytest.approx(0.7 * O.decode_bf16(q[0, t, h]) @ Kf[j, 0], rel=1e-15)
    # q = 0: uniform weights -> mean of the selected rows, lse = log(count)
    sel = np.array([3, 7, 8, 20, -1, -1])
    out, lse = O.sparse_attention_row(np.zeros((H_q, d)), Kf, Vf, sel, 1.0)
    assert np.allclose(out, Vf[[3, 7, 8, 20], 0].mean(axis=0)[None, :], rtol=1e-14, atol=1e-15)
    assert np.allclose(lse, math.log(4), rtol=1e-15)
    # empty selection: zero output, lse = -inf
    out, lse = O.sparse_attention_row(np.ones((H_q, d)), Kf, Vf, np.array([-1, -1]), 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    # order of the index list does not matter
    sel = rng.choice(S, size=12, replace=False)
    a, la = O.sparse_attention_row(O.decode_bf16(q[0, 0]), Kf, Vf, sel, 0.5)
    b, lb = O.sparse_attention_row(O.decode_bf16(q[0, 0]), Kf, Vf, sel[::-1].copy(), 0.5)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15) and np.allclose(la, lb, rtol=1e-14)


def test_attention_against_python_brute_force():
    rng = np.random.default_rng(12)
    T, S, H_q, H_kv, d = 3, 10, 4, 2, 8
    q, K, V = _attn_case(rng, T, S, H_q, H_kv, d)
    idx = np.array([[0, 4, 9, -1], [2, 3, -1, -1], [1, 5, 6, 7]])
    out, lse = O.sparse_attention_rows(q, K, V, idx, 0, [0, 1, 2], 0.35)
    qf, Kf, Vf = O.decode_bf16(q[0]), O.decode_bf16(K[0]), O.decode_bf16(V[0])
    for t in range(T):
        sel = [j for j in idx[t] if j >= 0]
        for h in range(H_q):
            g = h // (H_q // H_kv)
            lg = [0.35 * sum(qf[t, h, c] * Kf[j, g, c] for c in range(d)) for j in sel]
            z = sum(math.exp(x) for x in lg)
            for c in range(d):
                want = sum(math.exp(lg[i]) * Vf[j, g, c] for i, j in enumerate(sel)) / z
                assert out[t, h, c] == pytest.approx(want, rel=1e-12, abs=1e-13)
            assert lse[t, h] == pytest.approx(math.log(z), rel=1e-13, abs=1e-13)


# ---------------------------------------------------------------- IndexShare


def test_indexshare_selection_once_per_group(monkeypatch):
    g = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))["indexshare_group"]
    rng = np.random.default_rng(13)
    T, S, H, dI, k = 9, 9, 4, 64, 4
    ind = {"q_I": _rand_codes(rng, (1, T, H, dI)), "k_I": _rand_codes(rng, (1, S, dI)),
           "w": rng.random((1, T, H)).astype(np.float32), "q_pos0": np.array([0]),
           "kv_len": np.array([S])}
    layers = []
    for _ in range(g["group_layers"]):
        q, K, V = _attn_case(rng, T, S, 2, 1, 16)
        layers.append({"q": q, "K": K, "V": V})
    calls = {"n": 0}
    real = O.topk_rows

    def counting(*a, **kw):
        calls["n"] += 1
        return real(*a, **kw)

    monkeypatch.setattr(O, "topk_rows", counting)
    rows = list(range(T))
    idx, outs = O.indexshare_group(ind, layers, k, 0, rows, 0.25)
    assert calls["n"] == 1
    per_layer_calls = g["group_layers"]   # per-layer indexing runs it once per layer
    removed = 100 * (1 - calls["n"] / per_layer_calls)
    assert removed == g["indexer_cost_removed_percent"]
    for L, (out, lse) in zip(layers, outs):
        o2, l2 = O.sparse_attention_rows(L["q"], L["K"], L["V"], idx, 0, rows, 0.25)
        assert np.array_equal(out, o2) and np.array_equal(lse, l2)


# ---------------------------------------------------------------- IndexPool (reading)


def test_pool_keys_against_exact_mean():
    rng = np.random.default_rng(41)
    S, d_I, pool = 23, 16, 4
    codes = rng.integers(0, 256, (S, d_I)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38          # no NaN codes in a cache
    for kv_len in (23, 22, 9, 0):
        got = O.pool_keys(codes, kv_len, pool)
        assert got.shape == ((S + pool - 1) // pool, d_I)
        for j in range(got.shape[0]):
            rows = [s for s in range(pool * j, pool * j + pool) if s < min(S, kv_len)]
            for c in range(d_I):
                exact = sum((Fraction(float(O.E4M3_TABLE[codes[s, c]])) for s in rows),
                            Fraction(0)) / pool
                want = _nearest_e4m3_brute_force(float(exact)) if rows else 0
                assert got[j, c] == want, (kv_len, j, c)


def test_pooled_selection_with_pool_1_is_the_token_selection():
    rng = np.random.default_rng(42)
    S, H, d_I, k = 300, 4, 64, 20
    q = rng.integers(0, 256, (H, d_I)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    keys = rng.integers(0, 256, (S, d_I)).astype(np.uint8)
    keys[(keys & 0x7F) == 0x7F] = 0
    w = rng.uniform(0, 1, H)
    pooled = O.decode_e4m3(O.pool_keys(keys, S, 1))
    for t in (0, 5, 150, 299):
        n = O.visible_count(0, S, t)
        _, blocks, row = O.pooled_topk_row(q, pooled, w, 0, S, t, 1, k)
        want = O.select_topk(O.score_row(q, O.decode_e4m3(keys)[:n], w, n), k)
        assert np.array_equal(blocks, want) and np.array_equal(row, want)


def test_visible_blocks_brute_force():
    for pool in (1, 2, 4, 8):
        for pos0 in (-5, 0, 3, 17):
            for kv_len in (0, 1, 7, 30):
                for t in range(12):
                    p = pos0 + t
                    want = sum(1 for j in range(64) if pool * j <= p and pool * j < kv_len)
                    assert O.visible_blocks(pos0, kv_len, t, pool) == want


def test_pooled_selection_known_blocks_and_expansion():
    """Every block holds 4 copies of one key, so each block key is that key exactly and
    the block scores are known; a query whose position cuts the last block sees only its
    first tokens."""
    pool, nb, d_I = 4, 12, 64
    vals = [1.0 + 0.125 * i for i in range(8)] + [2.0, 2.25, 2.5, 2.75]   # e4m3 values
    order = [7, 2, 11, 0, 5, 9, 1, 3, 10, 4, 6, 8]            # block j gets vals[order[j]]
    keys = np.zeros((nb * pool, d_I), dtype=np.uint8)
    for j in range(nb):
        keys[pool * j: pool * j + pool, :] = int(np.nonzero(O.E4M3_TABLE == vals[order[j]])[0][0])
    pooled = O.decode_e4m3(O.pool_keys(keys, nb * pool, pool))
    assert np.all(pooled[:, 0] == np.array([vals[o] for o in order]))
    q = np.full((1, d_I), int(np.nonzero(O.E4M3_TABLE == 1.0)[0][0]), dtype=np.uint8)
    w = np.ones(1)
    pos0, t, kb = 42, 0, 3             # sees blocks 0..10, tokens 0..42 (block 10 cut at 42)
    sc, blocks, row = O.pooled_topk_row(q, pooled, w, pos0, nb * pool, t, pool, kb)
    assert len(sc) == 11
    best = sorted(range(11), key=lambda j: -order[j])[:kb]  # blocks 2, 10, 9
    assert blocks.tolist() == sorted(best)
    toks = [pool * j + r for j in sorted(best) for r in range(pool) if pool * j + r <= 42]
    assert row.tolist() == toks + [-1] * (kb * pool - len(toks))


# ---------------------------------------------------------------- attention backward


def _torch_bf16_bits(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_attention_backward_against_torch_autograd():
    """Dense attention with every unselected key masked out, differentiated by torch in
    fp64, gives the same gradients as the oracle's explicit chain rule."""
    g = torch.Generator().manual_seed(61)
    B, T, S, H_q, H_kv, d, k = 1, 6, 20, 4, 2, 8, 7
    q = torch.randn(B, T, H_q, d, generator=g)
    K = torch.randn(B, S, H_kv, d, generator=g)
    V = torch.randn(B, S, H_kv, d, generator=g)
    qb, Kb, Vb = _torch_bf16_bits(q), _torch_bf16_bits(K), _torch_bf16_bits(V)
    qf = torch.from_numpy(O.decode_bf16(qb)).requires_grad_()
    Kf = torch.from_numpy(O.decode_bf16(Kb)).requires_grad_()
    Vf = torch.from_numpy(O.decode_bf16(Vb)).requires_grad_()
    rng = np.random.default_rng(62)
    idx = np.full((T, k), -1)
    for t in range(T):
        n = rng.integers(1, k + 1)
        idx[t, :n] = np.sort(rng.choice(S, size=n, replace=False))
    mask = torch.full((T, S), float("-inf"), dtype=torch.float64)
    for t in range(T):
        mask[t, idx[t][idx[t] >= 0]] = 0.0
    scale = 0.37
    grp = H_q // H_kv
    outs = []
    for h in range(H_q):
        logits = scale * qf[0, :, h, :] @ Kf[0, :, h // grp, :].T + mask
        outs.append(torch.softmax(logits, dim=-1) @ Vf[0, :, h // grp, :])
    out = torch.stack(outs, dim=1)                      # [T, H_q, d]
    dout = torch.randn(T, H_q, d, generator=g, dtype=torch.float64)
    (out * dout).sum().backward()
    dq, dK, dV = O.sparse_attention_backward_rows(qb, Kb, Vb, idx, dout.numpy(), 0, list(range(T)),
                                                  scale)
    assert np.allclose(dq, qf.grad[0].numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dK, Kf.grad[0].numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dV, Vf.grad[0].numpy(), rtol=1e-10, atol=1e-12)


def test_attention_backward_finite_differences_and_closed_forms():
    rng = np.random.default_rng(63)
    S, H, d = 9, 1, 4
    K = rng.standard_normal((1, S, 1, d)).astype(np.float32)
    V = rng.standard_normal((1, S, 1, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    Kb, Vb, qb = (_torch_bf16_bits(torch.from_numpy(x)) for x in (K, V, q))
    idx = np.array([[1, 4, 6, -1]])
    dout = rng.standard_normal((1, H, d))
    dq, dK, dV = O.sparse_attention_backward_rows(qb, Kb, Vb, idx, dout, 0, [0], 0.5)
    # d/dq of sum(out * dout) by central differences on the decoded values
    qv = O.decode_bf16(qb)[0, 0, 0].copy()
    Kv, Vv = O.decode_bf16(Kb)[0], O.decode_bf16(Vb)[0]

    def f(qrow):
        o, _ = O.sparse_attention_row(qrow[None, :], Kv, Vv, idx[0], 0.5)
        return float((o[0] * dout[0, 0]).sum())
    eps = 1e-6
    num = np.array([(f(qv + eps * e) - f(qv - eps * e)) / (2 * eps) for e in np.eye(d)])
    assert np.allclose(dq[0, 0], num, rtol=1e-6, atol=1e-8)
    # one selected key: softmax is 1, so dq = 0, dK = 0 and dV = dout
    dq1, dK1, dV1 = O.sparse_attention_backward_rows(qb, Kb, Vb, np.array([[4, -1]]), dout, 0, [0], 0.5)
    assert np.all(dq1 == 0) and np.all(dK1 == 0)
    assert np.allclose(dV1[4, 0], dout[0, 0]) and np.all(np.delete(dV1, 4, axis=0) == 0)
    # unselected rows get no gradient; the dV rows sum to dout (the weights sum to 1)
    assert np.all(dK[[0, 2, 3, 5, 7, 8]] == 0) and np.all(dV[[0, 2, 3, 5, 7, 8]] == 0)
    assert np.allclose(dV[:, 0].sum(axis=0), dout[0, 0])


def test_attention_backward_magnitudes_by_enumeration():
    """Each magnitude is rebuilt with plain Python loops on a tiny input, product by product
    (dp_j = sum_c dO_c V_jc, D = sum_j p_j dp_j, a_j = sum_c |dO_c V_jc|), and the gradients
    never exceed their own "ds" (dq, dK) or "p" (dV) magnitudes (triangle inequality: they
    are exactly those sums taken with signs)."""
    rng = np.random.default_rng(64)
    T, S, H_q, H_kv, d, k = 3, 6, 4, 2, 3, 4
    q = rng.standard_normal((1, T, H_q, d)).astype(np.float32)
    K = rng.standard_normal((1, S, H_kv, d)).astype(np.float32)
    V = rng.standard_normal((1, S, H_kv, d)).astype(np.float32)
    qb, Kb, Vb = (_torch_bf16_bits(torch.from_numpy(x)) for x in (q, K, V))
    idx = np.array([[0, 2, 5, -1], [1, 2, 3, 4], [3, -1, -1, -1]])
    dout = rng.standard_normal((T, H_q, d))
    sc = -0.6
    m = O.sparse_attention_backward_magnitudes(qb, Kb, Vb, idx, dout, 0, list(range(T)), sc)
    qv, Kv, Vv = O.decode_bf16(qb)[0], O.decode_bf16(Kb)[0], O.decode_bf16(Vb)[0]
    bq = {n: np.zeros((T, H_q, d)) for n in ("ds", "dp", "dd", "da")}
    bk = {n: np.zeros((S, H_kv, d)) for n in ("ds", "dp", "dd")}
    bv = np.zeros((S, H_kv, d))
    grp = H_q // H_kv
    for t in range(T):
        sel = [int(j) for j in idx[t] if j >= 0]
        for h in range(H_q):
            g = h // grp
            lg = [sc * sum(float(qv[t, h, c]) * float(Kv[j, g, c]) for c in range(d)) for j in sel]
            ex = [math.exp(x - max(lg)) for x in lg]
            p = [e / sum(ex) for e in ex]
            dp = [sum(dout[t, h, c] * Vv[j, g, c] for c in range(d)) for j in sel]
            D = sum(pj * x for pj, x in zip(p, dp))
            a = [sum(abs(dout[t, h, c] * Vv[j, g, c]) for c in range(d)) for j in sel]
            A = sum(pj * x for pj, x in zip(p, a))
            for e in range(d):
                bq["ds"][t, h, e] = sum(abs(sc * p[i] * (dp[i] - D) * Kv[j, g, e])
                                        for i, j in enumerate(sel))
                bq["dp"][t, h, e] = sum(abs(sc * p[i] * a[i] * Kv[j, g, e]) for i, j in enumerate(sel))
                bq["dd"][t, h, e] = abs(sc) * A * abs(sum(p[i] * Kv[j, g, e] for i, j in enumerate(sel)))
                bq["da"][t, h, e] = sum(abs(sc * A * p[i] * Kv[j, g, e]) for i, j in enumerate(sel))
                for i, j in enumerate(sel):
                    bk["ds"][j, g, e] += abs(sc * p[i] * (dp[i] - D) * qv[t, h, e])
                    bk["dp"][j, g, e] += abs(sc * p[i] * a[i] * qv[t, h, e])
                    bk["dd"][j, g, e] += abs(sc * p[i] * A * qv[t, h, e])
                    bv[j, g, e] += abs(p[i] * dout[t, h, e])
    for n in bq:
        assert np.allclose(m["dq"][n], bq[n], rtol=1e-12, atol=1e-300), n
    for n in bk:
        assert np.allclose(m["dK"][n], bk[n], rtol=1e-12, atol=1e-300), n
    assert np.allclose(m["dV"]["p"], bv, rtol=1e-12, atol=1e-300)
    dq, dK, dV = O.sparse_attention_backward_rows(qb, Kb, Vb, idx, dout, 0, list(range(T)), sc)
    assert np.all(np.abs(dq) <= m["dq"]["ds"] * (1 + 1e-12))
    assert np.all(np.abs(dK) <= m["dK"]["ds"] * (1 + 1e-12))
    assert np.all(np.abs(dV) <= m["dV"]["p"] * (1 + 1e-12))
    # terms of one sign: with dout >= 0 every dV term is >= 0, so the magnitude is dV itself
    _, _, dVp = O.sparse_attention_backward_rows(qb, Kb, Vb, idx, np.abs(dout), 0, list(range(T)), sc)
    mp = O.sparse_attention_backward_magnitudes(qb, Kb, Vb, idx, np.abs(dout), 0, list(range(T)), sc)
    assert np.allclose(dVp, mp["dV"]["p"], rtol=1e-12, atol=0)
    # one kept key: p = 1, dl = 0, so "ds" vanishes and "dd" = "da" = s A |K|
    one = np.array([[2, -1, -1, -1]])
    m1 = O.sparse_attention_backward_magnitudes(qb, Kb, Vb, one, dout[:1], 0, [0], sc)
    assert np.all(m1["dq"]["ds"] == 0) and np.allclose(m1["dq"]["dd"], m1["dq"]["da"])


# ---------------------------------------------------------------- indexer KL objective (reading)


def test_indexer_kl_against_torch():
    """torch's kl_div on log-softmax of the scores and autograd for the score gradient."""
    g = torch.Generator().manual_seed(81)
    B, T, S, H_q, H_kv, d, k = 1, 5, 30, 4, 2, 8, 9
    q = torch.randn(B, T, H_q, d, generator=g)
    K = torch.randn(B, S, H_kv, d, generator=g)
    qb, Kb = _torch_bf16_bits(q), _torch_bf16_bits(K)
    rng = np.random.default_rng(82)
    idx = np.full((T, k), -1)
    for t in range(T):
        n = rng.integers(1, k + 1)
        idx[t, :n] = np.sort(rng.choice(S, size=n, replace=False))
    scores = rng.standard_normal((T, k)) * 3
    loss, dsc = O.indexer_kl_rows(qb, Kb, idx, scores, 0, list(range(T)), 0.4, S)
    qf, Kf = torch.from_numpy(O.decode_bf16(qb)), torch.from_numpy(O.decode_bf16(Kb))
    for t in range(T):
        sel = idx[t][idx[t] >= 0]
        tgt = torch.zeros(len(sel), dtype=torch.float64)
        for h in range(H_q):
            tgt += torch.softmax(0.4 * Kf[0, sel, h // 2, :] @ qf[0, t, h], dim=0)
        tgt /= H_q
        sc = torch.tensor(scores[t, :len(sel)], requires_grad=True)
        kl = torch.nn.functional.kl_div(torch.log_softmax(sc, dim=0), tgt, reduction="sum")
        kl.backward()
        assert abs(kl.item() - loss[t]) <= 1e-12 * max(1.0, abs(loss[t]))
        assert np.allclose(dsc[t, :len(sel)], sc.grad.numpy(), atol=1e-14)
        assert np.all(dsc[t, len(sel):] == 0)


def test_indexer_kl_closed_forms():
    rng = np.random.default_rng(83)
    S, H, d = 12, 2, 4
    K = rng.standard_normal((1, S, 1, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    Kb, qb = _torch_bf16_bits(torch.from_numpy(K)), _torch_bf16_bits(torch.from_numpy(q))
    idx = np.array([[2, 5, 7, -1]])
    # scores equal to the log of the target make the prediction equal to it: loss 0, gradient 0
    Kv, qv = O.decode_bf16(Kb)[0], O.decode_bf16(qb)[0, 0]
    tgt = np.zeros(3)
    for h in range(H):
        lg = 0.5 * (Kv[[2, 5, 7], 0, :] @ qv[h])
        e = np.exp(lg - lg.max())
        tgt += e / e.sum()
    tgt /= H
    scores = np.array([[*np.log(tgt) + 1.7, 0.0]])          # a shift changes nothing
    loss, dsc = O.indexer_kl_rows(qb, Kb, idx, scores, 0, [0], 0.5, S)
    assert abs(loss[0]) < 1e-12 and np.all(np.abs(dsc) < 1e-12)
    # one selected key: target = prediction = 1
    loss1, dsc1 = O.indexer_kl_rows(qb, Kb, np.array([[4, -1]]), np.array([[3.0, 9.0]]), 0, [0], 0.5, S)
    assert loss1[0] == 0 and np.all(dsc1 == 0)
    # an entry past kv_len is padding; an empty selection gives 0
    loss2, _ = O.indexer_kl_rows(qb, Kb, np.array([[11, -1]]), np.array([[1.0, 1.0]]), 0, [0], 0.5, 10)
    assert loss2[0] == 0


def test_indexer_kl_dense_lse_against_torch():
    """With the dense (all visible keys) lse, the target is the dense attention summed over
    heads, restricted to the kept keys and renormalised: built here with torch's softmax
    over the full causal row; the gradient from autograd."""
    g = torch.Generator().manual_seed(84)
    S, H_q, H_kv, d, k = 40, 8, 2, 16, 7
    q = torch.randn(1, 3, H_q, d, generator=g) * 2
    K = torch.randn(1, S, H_kv, d, generator=g)
    qb, Kb = _torch_bf16_bits(q), _torch_bf16_bits(K)
    qf, Kf = torch.from_numpy(O.decode_bf16(qb)), torch.from_numpy(O.decode_bf16(Kb))
    rng = np.random.default_rng(85)
    idx = np.stack([np.sort(rng.choice(S, size=k, replace=False)) for _ in range(3)])
    scores = rng.standard_normal((3, k))
    lse = np.zeros((3, H_q))
    tgts = []
    for t in range(3):
        dense = torch.zeros(S, dtype=torch.float64)
        for h in range(H_q):
            lg = 0.3 * Kf[0, :, h // 4, :] @ qf[0, t, h]
            lse[t, h] = torch.logsumexp(lg, 0).item()
            dense += torch.softmax(lg, 0)
        tg = dense[idx[t]]
        tgts.append(tg / tg.sum())
    loss, dsc = O.indexer_kl_rows(qb, Kb, idx, scores, 0, [0, 1, 2], 0.3, S, lse=lse)
    for t in range(3):
        sc = torch.tensor(scores[t], requires_grad=True)
        kl = torch.nn.functional.kl_div(torch.log_softmax(sc, 0), tgts[t], reduction="sum")
        kl.backward()
        assert abs(kl.item() - loss[t]) <= 1e-12 * max(1.0, abs(loss[t]))
        assert np.allclose(dsc[t], sc.grad.numpy(), atol=1e-14)
    # the sparse lse (over the kept keys) gives the default target
    sparse_lse = np.array([[torch.logsumexp(0.3 * Kf[0, idx[t], h // 4, :] @ qf[0, t, h], 0).item()
                            for h in range(H_q)] for t in range(3)])
    l1, d1 = O.indexer_kl_rows(qb, Kb, idx, scores, 0, [0, 1, 2], 0.3, S, lse=sparse_lse)
    l0, d0 = O.indexer_kl_rows(qb, Kb, idx, scores, 0, [0, 1, 2], 0.3, S)
    assert np.allclose(l1, l0, rtol=1e-12, atol=1e-15) and np.allclose(d1, d0, atol=1e-15)


# ---------------------------------------------------------------- indexer backward


def _torch_e4m3_codes(x):
    """fp32 tensor -> e4m3 bytes through torch's own cast (saturating first)."""
    return x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)


def _indexer_bwd_case(seed, B=2, T=6, S=40, H=8, dI=16, k=10):
    g = torch.Generator().manual_seed(seed)
    qI = _torch_e4m3_codes(torch.randn(B, T, H, dI, generator=g) * 2)
    kI = _torch_e4m3_codes(torch.randn(B, S, dI, generator=g))
    # exact zeros of x: head 0 of query 0 is all zero; head 1 reads only dimension 0,
    # which keys 0..9 of sequence 0 have at zero
    qI[0, 0, 0] = 0
    qI[0, 0, 1] = 0
    qI[0, 0, 1, 0] = _torch_e4m3_codes(torch.tensor([1.5]))[0]
    kI[0, :10, 0] = 0
    w = (torch.randn(B, T, H, generator=g)).numpy()
    rng = np.random.default_rng(seed)
    idx = np.full((B, T, k), -1)
    for b in range(B):
        for t in range(T):
            n = int(rng.integers(0, k + 1))
            idx[b, t, :n] = np.sort(rng.choice(S, size=n, replace=False))
    idx[0, 0, :3] = [0, 3, 7]   # keys whose x is 0 for head 1
    ds = rng.standard_normal((B, T, k))
    return qI, kI, w, idx, ds


def test_indexer_backward_against_torch_autograd():
    """Autograd of sum_j ds_j * score[idx_j] with the scores built densely in torch (e4m3
    decoded by torch's own float8 type); torch's ReLU gives gradient 0 at 0."""
    B, T, S = 2, 6, 40
    qI, kI, w, idx, ds = _indexer_bwd_case(91, B=B, T=T, S=S)
    kv_len = [S, 31]
    for b in range(B):
        Q = _torch_e4m3_values(qI[b]).requires_grad_(True)      # [T, H, d]
        Kt = _torch_e4m3_values(kI[b]).requires_grad_(True)     # [S, d]
        W = torch.tensor(w[b], dtype=torch.float64, requires_grad=True)
        X = torch.einsum("thd,sd->ths", Q, Kt)
        score = (W[:, :, None] * torch.relu(X)).sum(1)           # [T, S]
        loss = torch.zeros((), dtype=torch.float64)
        for t in range(T):
            for j in range(idx.shape[2]):
                s = int(idx[b, t, j])
                if 0 <= s < kv_len[b]:
                    loss = loss + float(ds[b, t, j]) * score[t, s]
        loss.backward()
        dq, dw, dk = O.indexer_backward_rows(qI, kI, w, idx[b], ds[b], b, list(range(T)), kv_len[b])
        scale = 1 + float(Q.grad.abs().max())
        assert np.allclose(dq, Q.grad.numpy(), rtol=0, atol=1e-12 * scale)
        assert np.allclose(dw, W.grad.numpy(), rtol=0, atol=1e-12 * (1 + float(W.grad.abs().max())))
        assert np.allclose(dk, Kt.grad.numpy(), rtol=0, atol=1e-12 * (1 + float(Kt.grad.abs().max())))
    # the planted zeros: head 0 of query 0 contributes nothing and gets no gradient
    dq, dw, _ = O.indexer_backward_rows(qI, kI, w, idx[0], ds[0], 0, [0], S)
    assert dw[0, 0] == 0 and np.all(dq[0, 0] == 0)


def test_indexer_backward_identities_and_finite_differences():
    """score is linear in w and positively homogeneous of degree 1 in q and in k, so
    <dw, w> = <dq, q> = <dk, k>; finite differences along directions that cross no zero
    of x; padding and empty selections."""
    T, S = 6, 40
    qI, kI, w, idx, ds = _indexer_bwd_case(92, B=1, T=T, S=S)
    rows = list(range(T))
    dq, dw, dk = O.indexer_backward_rows(qI, kI, w, idx[0], ds[0], 0, rows, S)
    q = O.decode_e4m3(qI[0])
    keys = O.decode_e4m3(kI[0])
    e_w = float(np.sum(dw * w[0]))
    e_q = float(np.sum(dq * q))
    e_k = float(np.sum(dk * keys))
    assert abs(e_q - e_w) <= 1e-10 * (1 + abs(e_w)) and abs(e_k - e_w) <= 1e-10 * (1 + abs(e_w))

    def loss(qv, kv, wv):
        tot = 0.0
        for t in rows:
            sel = idx[0, t][idx[0, t] >= 0]
            if sel.size:
                tot += float(ds[0, t, :sel.size] @ O.index_scores(qv[t], kv[sel], wv[t]))
        return tot

    rng = np.random.default_rng(93)
    eps = 1e-6
    for name, base, grad in (("q", q, dq), ("k", keys, dk), ("w", np.asarray(w[0], np.float64), dw)):
        d = rng.standard_normal(base.shape)
        if name == "q":   # keep the planted exact zeros of x fixed
            d[0, :2] = 0
        if name == "k":
            d[:10, 0] = 0
        args = {"q": q, "k": keys, "w": np.asarray(w[0], np.float64)}
        lp = loss(*[base + eps * d if n == name else args[n] for n in ("q", "k", "w")])
        lm = loss(*[base - eps * d if n == name else args[n] for n in ("q", "k", "w")])
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - float(np.sum(grad * d))) <= 1e-6 * (1 + abs(fd)), name

    # entries at or past kv_len are padding: the same as removing them
    cut = 25
    idx_cut = np.where(idx[0] < cut, idx[0], -1)
    a = O.indexer_backward_rows(qI, kI, w, idx[0], ds[0], 0, rows, cut)
    b_ = O.indexer_backward_rows(qI, kI, w, idx_cut, ds[0], 0, rows, S)
    for x, y in zip(a, b_):
        assert np.array_equal(x, y)
    # an empty selection gives zeros
    e = O.indexer_backward_rows(qI, kI, w, np.full((1, 10), -1), ds[0, :1], 0, [2], S)
    assert all(not np.any(x) for x in e)


def test_indexer_backward_through_the_kl_against_torch():
    """The KL's gradient carried into q_I, k_I and w: autograd of KL(target || softmax of
    the kept scores), with the target held fixed, equals indexer_kl_rows' dscores fed to
    indexer_backward_rows."""
    T, S, H_q, d = 4, 30, 2, 8
    qI, kI, w, idx, _ = _indexer_bwd_case(94, B=1, T=T, S=S, H=4, dI=16, k=8)
    g = torch.Generator().manual_seed(95)
    qa = _torch_bf16_bits(torch.randn(1, T, H_q, d, generator=g))
    Ka = _torch_bf16_bits(torch.randn(1, S, 1, d, generator=g))
    rows = list(range(T))
    Q = _torch_e4m3_values(qI[0]).requires_grad_(True)
    Kt = _torch_e4m3_values(kI[0]).requires_grad_(True)
    W = torch.tensor(w[0], dtype=torch.float64, requires_grad=True)
    score = (W[:, :, None] * torch.relu(torch.einsum("thd,sd->ths", Q, Kt))).sum(1)
    sel_scores = np.zeros(idx[0].shape)
    total = torch.zeros((), dtype=torch.float64)
    qf, Kf = torch.from_numpy(O.decode_bf16(qa)), torch.from_numpy(O.decode_bf16(Ka))
    for t in rows:
        sel = idx[0, t][idx[0, t] >= 0]
        if sel.size == 0:
            continue
        sel_scores[t, :sel.size] = score[t, sel].detach().numpy()
        tgt = sum(torch.softmax(0.5 * Kf[0, sel, 0, :] @ qf[0, t, h], 0) for h in range(H_q)) / H_q
        total = total + torch.nn.functional.kl_div(torch.log_softmax(score[t, sel], 0), tgt,
                                                   reduction="sum")
    total.backward()
    _, dsc = O.indexer_kl_rows(qa, Ka, idx[0], sel_scores, 0, rows, 0.5, S)
    dq, dw, dk = O.indexer_backward_rows(qI, kI, w, idx[0], dsc, 0, rows, S)
    assert np.allclose(dq, Q.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dw, W.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dk, Kt.grad.numpy(), rtol=0, atol=1e-12)
