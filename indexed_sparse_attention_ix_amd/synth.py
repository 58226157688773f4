"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

This module holds only random draws, the planted-key / key-drift construction and
the storage encodings (fp32 -> FP8 e4m3 bytes, fp32 -> bf16).  None of the path's
arithmetic (indexer scores, selection, attention) lives here.

Streams.  Every tensor comes from its own torch.Generator seeded from
(seed, stream id, layer) through numpy's SeedSequence:
  0 indexer queries q_I   1 indexer keys k_I   2 head weights w
  3 attention q           4 attention K        5 attention V
  6 planted positions     7 key-mean drift
Generation runs on the requested device; CPU and GPU generators give different (but
each fully seeded) numbers, so one test generates once and hands the same bytes to
both sides.

Recipe.
  * q_I, k_I ~ N(0,1) fp32, rounded to OCP e4m3 (round to nearest even, saturating to
    +-448; torch's cast after a clamp).
  * w ~ U(0,1) fp32.
  * q, K, V ~ N(0, qkv_std^2) fp32 rounded to bf16 (round to nearest even).
  * drift > 0: k_I[s] = z_s + m_{floor(s/1024)} with m_0 = 0 and
    m_{j+1} = m_j + eps_j, eps_j ~ N(0, drift^2 I).
  * planted = P > 0: for each query t, P positions drawn uniformly (with replacement)
    from its visible prefix [0, n_t) (all of them when n_t <= P), and
    q_I[t,h,:] += (4/sqrt(d_I)) * sum_{s in P_t} k_I[s,:] for every head h, using the
    already-rounded keys.  That lifts q.k_s by about 4 standard deviations
    (the std of q.k for unit-normal entries is sqrt(d_I)).
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np
import torch

from .workloads import Workload

E4M3_MAX = 448.0
ROW_CHUNK_ELEMS = 1 << 24  # fp32 elements drawn per chunk (bounds host memory)


def _gen(seed: int, stream: int, layer: int, device) -> torch.Generator:
    st = np.random.SeedSequence([seed, stream, layer]).generate_state(2, dtype=np.uint32)
    s = (int(st[0]) << 31) ^ int(st[1])
    g = torch.Generator(device=device)
    g.manual_seed(s & ((1 << 63) - 1))
    return g


def encode_e4m3(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> e4m3 bytes (uint8), nearest-even, saturating to +-448."""
    return x.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def decode_e4m3_torch(b: torch.Tensor) -> torch.Tensor:
    """e4m3 bytes -> fp32 through torch's own cast (used only for planting)."""
    return b.view(torch.float8_e4m3fn).to(torch.float32)


def _normal_rows(shape, g, device, std=1.0, mean_fn=None, encode=None):
    """Draw N(0, std^2) in leading-dim chunks and encode each chunk immediately."""
    lead = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    rows_per = max(1, ROW_CHUNK_ELEMS // max(inner, 1))
    out = None
    for r0 in range(0, lead, rows_per):
        r1 = min(lead, r0 + rows_per)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        if mean_fn is not None:
            x += mean_fn(r0, r1)
        y = encode(x) if encode is not None else x
        if out is None:
            out = torch.empty(tuple(shape), dtype=y.dtype, device=device)
        out[r0:r1] = y
        del x, y
    return out


def _key_drift(wl: Workload, layer: int, device) -> torch.Tensor:
    """Per-1024-key-block mean m_j, shape [B, nblk, d_I] (m_0 = 0)."""
    nblk = (wl.S + 1023) // 1024
    g = _gen(wl.seed, 7, layer, device)
    eps = torch.randn((wl.B, nblk, wl.d_I), generator=g, device=device) * wl.drift
    m = torch.zeros_like(eps)
    if nblk > 1:
        m[:, 1:] = torch.cumsum(eps[:, :-1], dim=1)
    return m


def indexer_inputs(wl: Workload, layer: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """FP8 indexer queries/keys, head weights and position metadata.

    Returns q_I uint8 [B,T,H_I,d_I], k_I uint8 [B,S,d_I], w fp32 [B,T,H_I],
    q_pos0 int32 [B], kv_len int32 [B].
    """
    device = torch.device(device)
    B, T, S, H, D = wl.B, wl.T, wl.S, wl.H_I, wl.d_I
    # keys: one row per token, shared by all indexer heads
    gk = _gen(wl.seed, 1, layer, device)
    k_I = torch.empty((B, S, D), dtype=torch.uint8, device=device)
    drift = _key_drift(wl, layer, device) if wl.drift > 0 else None
    for b in range(B):
        if drift is not None:
            db = drift[b]

            def mean_fn(r0, r1, db=db):
                blk = torch.arange(r0, r1, device=device) // 1024
                return db[blk]
        else:
            mean_fn = None
        k_I[b] = _normal_rows((S, D), gk, device, mean_fn=mean_fn, encode=encode_e4m3)

    # queries (with planting through the query side)
    gq = _gen(wl.seed, 0, layer, device)
    pos0 = torch.tensor(wl.pos0_list(), dtype=torch.int64, device=device)
    kvl = torch.tensor(wl.kv_len_list(), dtype=torch.int64, device=device)
    plant = None
    if wl.planted > 0:
        P = wl.planted
        gp = _gen(wl.seed, 6, layer, device)
        u = torch.rand((B, T, P), generator=gp, device=device, dtype=torch.float64)
        t_idx = torch.arange(T, device=device)
        n_t = torch.minimum(pos0[:, None] + t_idx[None, :] + 1, kvl[:, None]).clamp(min=0)
        pos = torch.floor(u * n_t[:, :, None].to(torch.float64)).to(torch.int64)
        small = n_t <= P  # fewer visible keys than plants: plant all of them
        ar = torch.arange(P, device=device)[None, None, :].expand(B, T, P)
        pos = torch.where(small[:, :, None], ar, pos)
        valid = torch.where(small[:, :, None], ar < n_t[:, :, None],
                            torch.ones_like(pos, dtype=torch.bool))
        pos = torch.where(valid, pos, torch.zeros_like(pos)).clamp(max=S - 1)
        plant = torch.zeros((B, T, D), dtype=torch.float32, device=device)
        for b in range(B):
            kb = decode_e4m3_torch(k_I[b])  # [S, D]
            rows = kb[pos[b].reshape(-1)].reshape(T, P, D)
            rows = rows * valid[b][:, :, None]
            plant[b] = rows.sum(dim=1) * (4.0 / math.sqrt(D))
            del kb, rows
    q_I = torch.empty((B, T, H, D), dtype=torch.uint8, device=device)
    for b in range(B):
        if plant is not None:
            pb = plant[b]

            def qmean(r0, r1, pb=pb):
                return pb[r0:r1, None, :]
        else:
            qmean = None
        q_I[b] = _normal_rows((T, H, D), gq, device, mean_fn=qmean, encode=encode_e4m3)

    gw = _gen(wl.seed, 2, layer, device)
    w = torch.rand((B, T, H), generator=gw, device=device, dtype=torch.float32)
    return {
        "q_I": q_I,
        "k_I": k_I,
        "w": w,
        "q_pos0": torch.tensor(wl.pos0_list(), dtype=torch.int32, device=device),
        "kv_len": torch.tensor(wl.kv_len_list(), dtype=torch.int32, device=device),
    }


def attention_inputs(wl: Workload, layer: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """bf16 attention q [B,T,H_q,d], K and V caches [B,S,H_kv,d] for one layer."""
    device = torch.device(device)
    bf = lambda x: x.to(torch.bfloat16)  # noqa: E731
    gq = _gen(wl.seed, 3, layer, device)
    gk = _gen(wl.seed, 4, layer, device)
    gv = _gen(wl.seed, 5, layer, device)
    q = torch.empty((wl.B, wl.T, wl.H_q, wl.d), dtype=torch.bfloat16, device=device)
    K = torch.empty((wl.B, wl.S, wl.H_kv, wl.d), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    for b in range(wl.B):
        q[b] = _normal_rows((wl.T, wl.H_q, wl.d), gq, device, std=wl.qkv_std, encode=bf)
        K[b] = _normal_rows((wl.S, wl.H_kv, wl.d), gk, device, std=wl.qkv_std, encode=bf)
        V[b] = _normal_rows((wl.S, wl.H_kv, wl.d), gv, device, std=wl.qkv_std, encode=bf)
    return {"q": q, "K": K, "V": V}


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
