"""GPU parity: the cache producer (ix_append_kv) against the oracle, bit for bit."""
import math

import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from oracle import ix_oracle as O
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _special_values():
    """Midpoints between neighbouring e4m3 magnitudes (and the floats either side), the
    subnormal range, saturation, signed zeros."""
    mags = sorted(set(abs(x) for x in O.E4M3_TABLE if not math.isnan(x)))
    v = []
    for lo, hi in zip(mags, mags[1:]):
        m = np.float32((lo + hi) / 2)
        v += [m, -m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    v += [0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 1e6, -1e30, 2.0 ** -10, -(2.0 ** -10),
          2.0 ** -12, 1e-30, -1e-30]
    return np.array(v, dtype=np.float32)


def _run(B, S, T_new, d_I, H_kv, d, pos0, seed, with_specials=False):
    say(f"[ix_append_kv] B={B} S={S} T_new={T_new} d_I={d_I} H_kv={H_kv} d={d} pos0={pos0}")
    g = torch.Generator(device="cpu").manual_seed(seed)
    kc = torch.randint(0, 256, (B, S, d_I), generator=g, dtype=torch.int32).to(torch.uint8)
    Kc = torch.randint(0, 1 << 16, (B, S, H_kv, d), generator=g, dtype=torch.int32).to(torch.int16)
    Vc = torch.randint(0, 1 << 16, (B, S, H_kv, d), generator=g, dtype=torch.int32).to(torch.int16)
    kn = (torch.randn((B, T_new, d_I), generator=g) * 8.0).float()
    if with_specials:
        sp = torch.from_numpy(_special_values())
        flat = kn.view(-1)
        n = min(flat.numel(), sp.numel())
        flat[:n] = sp[:n]
    Kn = torch.randint(0, 1 << 16, (B, T_new, H_kv, d), generator=g, dtype=torch.int32).to(torch.int16)
    Vn = torch.randint(0, 1 << 16, (B, T_new, H_kv, d), generator=g, dtype=torch.int32).to(torch.int16)
    p0 = torch.tensor(pos0, dtype=torch.int32)

    dev = [t.to(DEV) for t in (kc, Kc, Vc, kn, Kn, Vn, p0)]
    dkc, dKc, dVc, dkn, dKn, dVn, dp0 = dev
    bd.append_kv(dp0, k_I_new=dkn, k_I_cache=dkc, K_new=dKn.view(torch.bfloat16),
                 V_new=dVn.view(torch.bfloat16), K_cache=dKc.view(torch.bfloat16),
                 V_cache=dVc.view(torch.bfloat16))
    torch.cuda.synchronize()
    rk, rK, rV = O.append_kv(kc.numpy(), Kc.numpy().view(np.uint16), Vc.numpy().view(np.uint16),
                             kn.numpy(), Kn.numpy().view(np.uint16), Vn.numpy().view(np.uint16),
                             p0.numpy())
    gk = dkc.cpu().numpy()
    nan_code = lambda c: (c & 0x7F) == 0x7F  # noqa: E731
    assert np.array_equal(nan_code(gk), nan_code(rk))
    both = ~nan_code(rk)
    assert np.array_equal(gk[both], rk[both])
    assert np.array_equal(dKc.cpu().numpy().view(np.uint16), rK)
    assert np.array_equal(dVc.cpu().numpy().view(np.uint16), rV)


def test_append_decode_token_with_special_values():
    _run(B=5, S=40, T_new=1, d_I=128, H_kv=1, d=128, pos0=[0, 39, 17, 40, -3], seed=31,
         with_specials=True)


def test_append_prefill_chunk_ragged_positions():
    # a chunk that runs past the end of one cache, d_I = 64, several KV heads
    _run(B=3, S=300, T_new=37, d_I=64, H_kv=2, d=64, pos0=[0, 280, 100], seed=32,
         with_specials=True)


def test_append_nan_gives_nan_code():
    kn = torch.full((1, 1, 64), float("nan"), device=DEV)
    kc = torch.zeros((1, 4, 64), dtype=torch.uint8, device=DEV)
    bd.append_kv(torch.tensor([2], dtype=torch.int32, device=DEV), k_I_new=kn, k_I_cache=kc)
    torch.cuda.synchronize()
    row = kc[0, 2].cpu().numpy()
    assert np.all((row & 0x7F) == 0x7F)
    assert np.all(kc[0, [0, 1, 3]].cpu().numpy() == 0)


def test_append_decode_size_cache_in_place():
    """One new token per sequence into 64 caches of 131072 positions (the decode shape);
    the written rows match the oracle and a sample of other rows is untouched."""
    B, S, d_I, H_kv, d = 64, 131072, 128, 1, 128
    say(f"[ix_append_kv] decode-size B={B} S={S}")
    g = torch.Generator(device=DEV).manual_seed(33)
    kc = torch.randint(0, 256, (B, S, d_I), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    Kc = torch.randn((B, S, H_kv, d), generator=g, device=DEV).to(torch.bfloat16)
    Vc = torch.randn((B, S, H_kv, d), generator=g, device=DEV).to(torch.bfloat16)
    before = [t[:, ::997].clone() for t in (kc, Kc, Vc)]
    pos = torch.randint(0, S, (B,), generator=g, device=DEV, dtype=torch.int32)
    kn = torch.randn((B, 1, d_I), generator=g, device=DEV) * 4.0
    Kn = torch.randn((B, 1, H_kv, d), generator=g, device=DEV).to(torch.bfloat16)
    Vn = torch.randn((B, 1, H_kv, d), generator=g, device=DEV).to(torch.bfloat16)
    bd.append_kv(pos, k_I_new=kn, k_I_cache=kc, K_new=Kn, V_new=Vn, K_cache=Kc, V_cache=Vc)
    torch.cuda.synchronize()
    p = pos.long()
    bidx = torch.arange(B, device=DEV)
    want = O.encode_e4m3(kn[:, 0].cpu().numpy())
    assert np.array_equal(kc[bidx, p].cpu().numpy(), want)
    assert torch.equal(Kc[bidx, p], Kn[:, 0]) and torch.equal(Vc[bidx, p], Vn[:, 0])
    # untouched rows of the sample (positions that are not this sequence's new token)
    cols = torch.arange(0, S, 997, device=DEV)
    keep = cols[None, :] != p[:, None]
    for t, b0 in zip((kc, Kc, Vc), before):
        now = t[:, ::997]
        assert torch.equal(now[keep], b0[keep])
