"""The MFMA error bounds the tolerances rest on, measured through the C ABI and asserted with
a factor-2 margin.

Tolerances built on them: scores near zero and the indexer backward's dw (FP8_MFMA_REL), the
attention backward and the indexer backward's dq_I and dk_I (BF16_MFMA_REL); and the indexer
backward kernel decides its ReLU mask exactly by recomputing every FP8 dot product within
FP8_MASK_WINDOW |q|_2 |k|_2 of zero, which is exact only if the FP8 MFMA error stays below that.

Two calls expose single dot products with nothing else rounded:
  * ix_score with one-hot head weights: each score is max(0, x) for one FP8 dot product x,
    times 1 and plus zeros, so |score - max(0, x_exact)| <= |x_gpu - x_exact|;
  * sparse_attn_fwd with one kept key per query: lse = sm_scale q.K_j, formed from the bf16
    MFMA dot product by three fp32 multiplications (by fl(sm_scale log2 e) and by ln 2),
    which add at most 6 2^-24 |lse|.
The FP8 inputs cover codes over the whole e4m3 range (the worst case seen: products of mixed
sign and very different size), N(0,1) codes as in the workloads, and one dominant product
among small ones of mixed sign.
"""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from oracle import ix_oracle as O
from parity_util import BF16_MFMA_REL, FP8_MASK_WINDOW, FP8_MFMA_REL, FP32_U, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _codes(rng, shape, lo=0, hi=256):
    c = rng.integers(lo, hi, size=shape, dtype=np.uint32).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E   # no NaN codes
    return c


def _fp8_case(kind, d_I, rng, T=256, S=2048, H=16):
    if kind == "full range":
        q, k = _codes(rng, (1, T, H, d_I)), _codes(rng, (1, S, d_I))
    elif kind == "normal":
        q = O.encode_e4m3(rng.standard_normal((1, 64, H, d_I)))
        k = O.encode_e4m3(rng.standard_normal((1, S, d_I)))
    else:  # one dominant product (448 * 448) among small products of both signs
        q = _codes(rng, (1, T, H, d_I), 0x08, 0x40) | (rng.integers(0, 2, (1, T, H, d_I)) << 7).astype(np.uint8)
        k = _codes(rng, (1, S, d_I), 0x08, 0x40)
        q[..., 0] = 0x7E
        k[..., 0] = 0x7E
    return q, k


@pytest.mark.parametrize("d_I", [64, 128])
def test_fp8_mfma_error_within_half_the_bounds(d_I):
    rng = np.random.default_rng(81 + d_I)
    worst_sum = worst_l2 = 0.0
    for kind in ("full range", "normal", "dominant"):
        q, k = _fp8_case(kind, d_I, rng)
        T, H, S = q.shape[1], q.shape[2], k.shape[1]
        w = np.zeros((1, T, H), dtype=np.float32)
        w[0, np.arange(T), np.arange(T) % H] = 1.0
        sc = bd.score(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                      torch.from_numpy(w).to(DEV),
                      torch.tensor([S - 1], dtype=torch.int32, device=DEV),
                      torch.tensor([S], dtype=torch.int32, device=DEV)).cpu().numpy()[0]
        qv = O.decode_e4m3(q[0])[np.arange(T), np.arange(T) % H]      # [T, d_I] the weighted head
        kv = O.decode_e4m3(k[0])
        x = qv @ kv.T                                                 # exact (multiples of 2^-18)
        err = np.abs(sc.astype(np.float64) - np.maximum(x, 0.0))
        mag = np.abs(qv) @ np.abs(kv).T
        l2 = np.linalg.norm(qv, axis=1)[:, None] * np.linalg.norm(kv, axis=1)[None, :]
        assert np.all(err[mag == 0] == 0)
        r_sum = float((err / np.maximum(mag, 1e-300)).max())
        r_l2 = float((err / np.maximum(l2, 1e-300)).max())
        say(f"[FP8 MFMA error] d_I={d_I} {kind}: {T} x {S} dot products; worst err / sum|q k| "
            f"{r_sum:.3e}, err / (|q| |k|) {r_l2:.3e}")
        worst_sum, worst_l2 = max(worst_sum, r_sum), max(worst_l2, r_l2)
    assert worst_sum <= FP8_MFMA_REL / 2, f"FP8 MFMA error ratio {worst_sum:.3e} within 2x of the bound"
    assert worst_l2 <= FP8_MASK_WINDOW / 2, \
        f"FP8 MFMA error {worst_l2:.3e} |q||k| within 2x of the backward's exact-mask window"


@pytest.mark.parametrize("d_I", [64, 128])
def test_64_head_scores_within_half_the_bound(d_I):
    """At 64 heads the indexer takes the head sum as 1/2 sum w|x| plus one MFMA of the keys with
    u = sum_h w_h q_h split into four scaled e4m3 terms.  Its error against the exact score,
    relative to N = sum_h w_h sum_c |q_hc k_c|, must stay within half of FP8_MFMA_REL too, on
    the same three kinds of codes, with dense weights (u then spans a wide range)."""
    rng = np.random.default_rng(91 + d_I)
    H, T, S = 64, 64, 2048
    worst = 0.0
    for kind in ("full range", "normal", "dominant"):
        q, k = _fp8_case(kind, d_I, rng, T=T, S=S, H=H)
        T_ = q.shape[1]
        w = rng.uniform(0.0, 1.0, (1, T_, H)).astype(np.float32)
        sc = bd.score(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                      torch.from_numpy(w).to(DEV),
                      torch.tensor([S - 1], dtype=torch.int32, device=DEV),
                      torch.tensor([S], dtype=torch.int32, device=DEV)).cpu().numpy()[0]
        qv = O.decode_e4m3(q[0])                                       # [T, H, d_I]
        kv = O.decode_e4m3(k[0])                                       # [S, d_I]
        wd = w[0].astype(np.float64)
        x = np.einsum("thc,sc->ths", qv, kv)                           # exact
        exact = np.einsum("th,ths->ts", wd, np.maximum(x, 0.0))
        mag = np.einsum("th,thc->tc", wd, np.abs(qv)) @ np.abs(kv).T
        err = np.abs(sc.astype(np.float64) - exact)
        r = float((err / np.maximum(mag, 1e-300)).max())
        say(f"[64-head scores] d_I={d_I} {kind}: {T_} x {S} scores; worst err / N {r:.3e}")
        worst = max(worst, r)
    assert worst <= FP8_MFMA_REL / 2, f"64-head score error ratio {worst:.3e} within 2x of the bound"


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_mfma_error_within_half_the_bound(d):
    g = torch.Generator(device="cpu").manual_seed(83 + d)
    T, S, H_q = 2048, 4096, 16
    # magnitudes spread over several binades, so products align at different exponents
    q = torch.randn(1, T, H_q, d, generator=g) * torch.exp2(torch.randint(-6, 7, (1, T, H_q, d),
                                                                          generator=g).float())
    K = torch.randn(1, S, 1, d, generator=g) * torch.exp2(torch.randint(-6, 7, (1, S, 1, d),
                                                                        generator=g).float())
    q, K = q.to(torch.bfloat16), K.to(torch.bfloat16)
    V = torch.zeros(1, S, 1, d, dtype=torch.bfloat16)
    sel = torch.randint(0, S, (1, T, 1), generator=g, dtype=torch.int32)
    scale = d ** -0.5
    _, lse = bd.sparse_attention(q.to(DEV), K.to(DEV), V.to(DEV), sel.to(DEV), scale,
                                 with_lse=True)
    lse = lse.cpu().numpy()[0].astype(np.float64)                 # [T, H_q]
    qf = q.double().numpy()[0]
    Ks = K.double().numpy()[0, :, 0][sel.numpy()[0, :, 0]]        # [T, d]
    exact = scale * np.einsum("thd,td->th", qf, Ks)
    mag = scale * np.einsum("thd,td->th", np.abs(qf), np.abs(Ks))
    err = np.maximum(np.abs(lse - exact) - 6 * FP32_U * np.abs(exact), 0.0)
    worst = float((err / mag).max())
    say(f"[bf16 MFMA error] d={d}: {T * H_q} dot products through sparse_attn_fwd lse (k = 1); "
        f"worst err / sum|q K| {worst:.3e}")
    assert worst <= BF16_MFMA_REL / 2, f"bf16 MFMA error ratio {worst:.3e} within 2x of the bound"
