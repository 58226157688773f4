"""GPU: the library's debug status (ix_debug_enable / ix_debug_read).

- Selection entries that name no key (outside [-1, kv_len)) are counted exactly, once per
  call that takes a selection from the caller, and not while the status is off.
- Turning the status on changes no result (the top-k, the attention and the backward are
  bitwise the same).
- The top-k's counters: a query that sees more keys than a candidate buffer holds, with no
  threshold sample to start from, must compact its buffer; no entry is ever dropped for lack
  of room.
"""
import numpy as np
import pytest
import torch

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import synth
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _debug_off_after():
    yield
    bd.ix_debug_enable(0)


def _attn_case(seed, B=2, T=24, S=300, H_q=16, H_kv=1, d=128, k=64, kv_lens=(300, 150)):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = (torch.randn(B, T, H_q, d, generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    K = (torch.randn(B, S, H_kv, d, generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    V = torch.randn(B, S, H_kv, d, generator=g).to(torch.bfloat16).to(DEV)
    kvl = np.array(kv_lens, dtype=np.int32)
    rng = np.random.default_rng(seed)
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            n = int(rng.integers(1, k + 1))
            idx[b, t, :n] = np.sort(rng.choice(int(kvl[b]), size=n, replace=False))
    # planted entries that name no key: below the padding value, at or past kv_len, past S
    flat = idx.reshape(-1)
    pos = rng.choice(flat.size, size=97, replace=False)
    bad = np.array([-2, -1000, 10 ** 6, 299, 300, 150, 151], dtype=np.int32)
    flat[pos] = bad[rng.integers(0, bad.size, size=pos.size)]
    kvl_b = np.repeat(kvl, T * k).reshape(idx.shape)
    expected = int(((idx < -1) | (idx >= kvl_b)).sum())
    return q, K, V, idx, kvl, expected


def test_out_of_range_entries_counted_per_call():
    q, K, V, idx, kvl, expected = _attn_case(301)
    say(f"[debug status] {expected} entries of the selection name no key")
    assert expected > 50
    didx = torch.from_numpy(idx).to(DEV)
    dkvl = torch.from_numpy(kvl).to(DEV)
    d = q.shape[-1]
    scale = d ** -0.5

    bd.ix_debug_enable(1)
    bd.ix_debug_read(reset=1)
    out, lse = bd.sparse_attention(q, K, V, didx, scale, kv_len=dkvl, with_lse=True)
    st = bd.ix_debug_read(reset=1)
    assert st["idx_out_of_range"] == expected, st
    # three layers over one selection: one pass over it
    bd.group_attention([{"q": q, "K": K, "V": V}] * 3, didx, scale, kv_len=dkvl)
    assert bd.ix_debug_read(reset=1)["idx_out_of_range"] == expected
    dout = torch.randn(q.shape, generator=torch.Generator(device="cpu").manual_seed(7)).to(
        torch.bfloat16).to(DEV)
    bd.sparse_attention_backward(q, K, V, didx, out, lse, dout, scale, kv_len=dkvl)
    bd.sparse_attention_backward(q, K, V, didx, out, lse, dout, scale, kv_len=dkvl, rows_per_pass=5)
    assert bd.ix_debug_read(reset=1)["idx_out_of_range"] == 2 * expected
    sel = torch.randn(idx.shape, generator=torch.Generator(device="cpu").manual_seed(8)).to(DEV)
    bd.indexer_kl(q, K, didx, lse, sel, scale, kv_len=dkvl)
    assert bd.ix_debug_read(reset=1)["idx_out_of_range"] == expected
    # the indexer backward takes kv_len from the indexer arguments
    B, T, k = idx.shape
    S = K.shape[1]
    g = torch.Generator(device="cpu").manual_seed(9)
    qI = synth.encode_e4m3(torch.randn(B, T, 8, 64, generator=g)).to(DEV)
    kI = synth.encode_e4m3(torch.randn(B, S, 64, generator=g)).to(DEV)
    w = torch.randn(B, T, 8, generator=g).to(DEV)
    args = bd.indexer_args(qI, kI, w, torch.zeros(B, dtype=torch.int32, device=DEV), dkvl)
    bd.indexer_bwd(args, didx, sel, DEV)
    assert bd.ix_debug_read(reset=1)["idx_out_of_range"] == expected
    # off: nothing is counted
    bd.ix_debug_enable(0)
    bd.sparse_attention(q, K, V, didx, scale, kv_len=dkvl)
    torch.cuda.synchronize()
    assert bd.ix_debug_read()["idx_out_of_range"] == 0


def test_debug_status_changes_no_result():
    say("[debug status] results with the status on and off")
    g = torch.Generator(device="cpu").manual_seed(302)
    B, T, S, H_I, d_I, k = 1, 64, 2000, 64, 128, 64
    qI = synth.encode_e4m3(torch.randn(B, T, H_I, d_I, generator=g)).to(DEV)
    kI = synth.encode_e4m3(torch.randn(B, S, d_I, generator=g)).to(DEV)
    w = torch.randn(B, T, H_I, generator=g).to(DEV)
    pos0 = torch.tensor([S - T], dtype=torch.int32, device=DEV)
    kvl = torch.tensor([S], dtype=torch.int32, device=DEV)
    q, K, V, idx_a, kvl_a, _ = _attn_case(303)
    didx = torch.from_numpy(idx_a).to(DEV)
    dkvl = torch.from_numpy(kvl_a).to(DEV)
    runs = []
    for on in (0, 1, 0):
        bd.ix_debug_enable(on)
        sel_idx, sel = bd.topk(qI, kI, w, pos0, kvl, k, with_scores=True)
        out, lse = bd.sparse_attention(q, K, V, didx, q.shape[-1] ** -0.5, kv_len=dkvl, with_lse=True)
        torch.cuda.synchronize()
        runs.append([x.clone() for x in (sel_idx, sel, out, lse)])
    for r in runs[1:]:
        for x, y in zip(runs[0], r):
            assert torch.equal(x, y)


def test_topk_counters():
    """64 queries at the end of 2000 keys, 64 heads, k = 64: a unit of 125 key tiles is too
    short for a threshold sample (at least 4 tiles per sampled tile), so every visible key
    enters its query's candidate buffer (1152 entries) until the buffer compacts: each query
    compacts at least once.  No entry is dropped for lack of room, in this case or at 128
    queries over 70,000 keys with key splits."""
    say("[debug status] top-k counters")
    bd.ix_debug_enable(1)
    bd.ix_debug_read(reset=1)
    g = torch.Generator(device="cpu").manual_seed(304)
    B, T, S, H_I, d_I, k = 1, 64, 2000, 64, 128, 64
    qI = synth.encode_e4m3(torch.randn(B, T, H_I, d_I, generator=g)).to(DEV)
    kI = synth.encode_e4m3(torch.randn(B, S, d_I, generator=g)).to(DEV)
    w = torch.randn(B, T, H_I, generator=g).to(DEV)
    pos0 = torch.tensor([S - T], dtype=torch.int32, device=DEV)
    kvl = torch.tensor([S], dtype=torch.int32, device=DEV)
    bd.topk(qI, kI, w, pos0, kvl, k)
    st = bd.ix_debug_read(reset=1)
    say(f"  {st}")
    assert st["topk_compactions"] >= T
    assert st["topk_overflow"] == 0 and st["idx_out_of_range"] == 0
    # decode-like: few queries, many keys, so the keys split across units and merge
    B, T, S, k = 2, 2, 70000, 2048
    qI = synth.encode_e4m3(torch.randn(B, T, H_I, d_I, generator=g)).to(DEV)
    kI = synth.encode_e4m3(torch.randn(B, S, d_I, generator=g)).to(DEV)
    w = torch.randn(B, T, H_I, generator=g).to(DEV)
    pos0 = torch.tensor([S - T, S - 40000], dtype=torch.int32, device=DEV)
    kvl = torch.tensor([S, S - 40000 + T], dtype=torch.int32, device=DEV)
    bd.topk(qI, kI, w, pos0, kvl, k)
    st = bd.ix_debug_read(reset=1)
    say(f"  {st}")
    assert st["topk_overflow"] == 0
