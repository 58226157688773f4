"""C-ABI library on the host (no GPU): it loads, exports every declared symbol, sizes
workspaces, and rejects invalid arguments before launching anything."""
import ctypes
import os
import re

import pytest

from indexed_sparse_attention_ix_amd import binding as bd
from indexed_sparse_attention_ix_amd import peaks as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

pytestmark = pytest.mark.skipif(not os.path.exists(bd.LIB_PATH), reason="libix.so not built")


def declared_functions(header):
    text = open(os.path.join(INCLUDE, header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    # ix.h is libix.so's interface; ix_peaks.h is the microbenchmark library's
    assert sorted(f for f in os.listdir(INCLUDE) if f.endswith(".h")) == ["ix.h", "ix_peaks.h"]
    names = declared_functions("ix.h")
    assert set(names) == set(bd.EXPORTS)
    lib = ctypes.CDLL(bd.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert not any(hasattr(lib, n) for n in pk.EXPORTS), "microbenchmarks in the path's library"
    pnames = declared_functions("ix_peaks.h")
    assert set(pnames) == set(pk.EXPORTS)
    plib = ctypes.CDLL(pk.LIB_PATH)
    for n in pnames:
        assert hasattr(plib, n), n


def test_abi_version_and_clean_error():
    assert bd.ix_abi_version() == bd.ABI_VERSION == 5


FAKE = 1 << 20  # 16-byte aligned non-null stand-in address; never dereferenced on failure


def args(**kw):
    d = dict(q=FAKE, k=FAKE, w=FAKE, q_pos0=FAKE, kv_len=FAKE, B=1, T=128, S_max=128, H_I=64,
             d_I=128)
    d.update(kw)
    return bd.IndexerArgs(d["q"], d["k"], d["w"], d["q_pos0"], d["kv_len"], d["B"], d["T"],
                          d["S_max"], d["H_I"], d["d_I"])


def status_of(fn, *a):
    try:
        fn(*a)
    except bd.IxError as e:
        return e.status
    return bd.IX_OK


def test_indexer_validation_codes():
    L = bd.load()
    assert L.ix_topk(None, 64, FAKE, None, FAKE, 1 << 30, None) == bd.IX_ERR_INVALID
    assert "NULL" in bd.ix_last_error()
    assert status_of(bd.ix_topk, args(d_I=96), 64, FAKE, 0, FAKE, 1 << 30) == bd.IX_ERR_UNSUPPORTED
    assert status_of(bd.ix_topk, args(H_I=6), 64, FAKE, 0, FAKE, 1 << 30) == bd.IX_ERR_UNSUPPORTED
    assert status_of(bd.ix_topk, args(H_I=68), 64, FAKE, 0, FAKE, 1 << 30) == bd.IX_ERR_UNSUPPORTED
    assert status_of(bd.ix_topk, args(), 0, FAKE, 0, FAKE, 1 << 30) == bd.IX_ERR_UNSUPPORTED
    assert status_of(bd.ix_topk, args(), 4096, FAKE, 0, FAKE, 1 << 30) == bd.IX_ERR_UNSUPPORTED
    assert status_of(bd.ix_topk, args(B=-1), 64, FAKE, 0, FAKE, 1 << 30) == bd.IX_ERR_INVALID
    assert status_of(bd.ix_topk, args(w=0), 64, FAKE, 0, FAKE, 1 << 30) == bd.IX_ERR_INVALID
    assert status_of(bd.ix_topk, args(q=FAKE + 8), 64, FAKE, 0, FAKE, 1 << 30) == bd.IX_ERR_INVALID
    assert status_of(bd.ix_topk, args(), 64, 0, 0, FAKE, 1 << 30) == bd.IX_ERR_INVALID
    need = bd.ix_topk_workspace_bytes(args(), 64)
    assert need > 0
    assert status_of(bd.ix_topk, args(), 64, FAKE, 0, FAKE, need - 1) == bd.IX_ERR_WORKSPACE
    assert status_of(bd.ix_topk, args(), 64, FAKE, 0, 0, need) == bd.IX_ERR_WORKSPACE
    assert "workspace" in bd.ix_last_error()
    # ix_score row range
    assert status_of(bd.ix_score, args(), -1, 4, FAKE) == bd.IX_ERR_INVALID
    assert status_of(bd.ix_score, args(), 5, 4, FAKE) == bd.IX_ERR_INVALID
    assert status_of(bd.ix_score, args(), 0, 129, FAKE) == bd.IX_ERR_INVALID
    assert status_of(bd.ix_score, args(), 0, 4, 0) == bd.IX_ERR_INVALID


def test_empty_calls_launch_nothing():
    # B == 0 or T == 0: OK without touching any pointer
    assert status_of(bd.ix_topk, args(B=0, q=0, k=0, w=0, q_pos0=0, kv_len=0), 64, 0, 0, 0, 0) == bd.IX_OK
    assert status_of(bd.ix_topk, args(T=0, q=0, k=0, w=0, q_pos0=0, kv_len=0), 64, 0, 0, 0, 0) == bd.IX_OK
    assert status_of(bd.ix_score, args(T=0), 0, 0, 0) == bd.IX_OK
    assert status_of(bd.ix_score, args(), 3, 3, 0) == bd.IX_OK
    assert bd.ix_topk_workspace_bytes(args(B=0), 64) == 0
    assert status_of(bd.sparse_attn_fwd, 0, 0, 0, 0, 0, 0, 5, 100, 16, 1, 128, 64, 0.1, 0, 0,
                     0, 0) == bd.IX_OK


def test_attention_validation_codes():
    ok = dict(q=FAKE, kc=FAKE, vc=FAKE, idx=FAKE, kv_len=0, B=1, T=4, S_max=64, H_q=16, H_kv=1,
              d=128, k=64, sm_scale=0.1, out=FAKE, lse=0, ws=0, ws_bytes=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return status_of(bd.sparse_attn_fwd, a["q"], a["kc"], a["vc"], a["idx"], a["kv_len"],
                         a["B"], a["T"], a["S_max"], a["H_q"], a["H_kv"], a["d"], a["k"],
                         a["sm_scale"], a["out"], a["lse"], a["ws"], a["ws_bytes"])

    assert call(d=96) == bd.IX_ERR_UNSUPPORTED
    assert call(H_q=12, H_kv=5) == bd.IX_ERR_UNSUPPORTED
    assert call(H_q=32, H_kv=1) == bd.IX_ERR_UNSUPPORTED
    assert call(k=0) == bd.IX_ERR_UNSUPPORTED
    assert call(T=-1) == bd.IX_ERR_INVALID
    assert call(out=0) == bd.IX_ERR_INVALID
    assert call(kc=FAKE + 2) == bd.IX_ERR_INVALID
    assert call(sm_scale=float("nan")) == bd.IX_ERR_INVALID
    # one sequence's K/V cache is addressed with 32-bit buffer offsets: at most 2 GiB
    assert call(S_max=(1 << 23) + 1, H_kv=1, H_q=16) == bd.IX_ERR_UNSUPPORTED
    assert call(S_max=1 << 20, H_kv=16, H_q=16) == bd.IX_ERR_UNSUPPORTED
    # decode-sized batches split the selection and need a workspace
    need = bd.sparse_attn_workspace_bytes(64, 1, 16, 1, 128, 2048)
    assert need > 0
    assert call(B=64, T=1, k=2048) == bd.IX_ERR_WORKSPACE
    assert bd.sparse_attn_workspace_bytes(1, 4096, 16, 1, 128, 2048) == 0


def test_indexshare_validation_codes():
    a = args()
    L = bd.load()
    P = ctypes.POINTER(ctypes.c_void_p)
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    pa = ctypes.cast(arr, P)
    need = bd.indexshare_workspace_bytes(a, 64, 16, 1, 128)
    assert need >= bd.ix_topk_workspace_bytes(a, 64)
    assert L.indexshare_group_fwd(ctypes.byref(a), 64, 0, pa, pa, pa, pa, None, 16, 1, 128,
                                  ctypes.c_float(0.1), FAKE, FAKE, need, None) == bd.IX_ERR_INVALID
    assert L.indexshare_group_fwd(ctypes.byref(a), 64, 4, None, pa, pa, pa, None, 16, 1, 128,
                                  ctypes.c_float(0.1), FAKE, FAKE, need, None) == bd.IX_ERR_INVALID
    assert L.indexshare_group_fwd(ctypes.byref(a), 64, 4, pa, pa, pa, pa, None, 16, 1, 128,
                                  ctypes.c_float(0.1), FAKE, FAKE, need - 1, None) == bd.IX_ERR_WORKSPACE
    assert L.indexshare_group_fwd(ctypes.byref(a), 64, 4, pa, pa, pa, pa, None, 16, 1, 96,
                                  ctypes.c_float(0.1), FAKE, FAKE, need, None) == bd.IX_ERR_UNSUPPORTED


def test_noalloc_validation_codes():
    # the no-allocation group call validates like indexshare_group_fwd and refuses, before
    # looking up its scratch or launching, a call whose workspace would exceed the scratch
    L = bd.load()
    P = ctypes.POINTER(ctypes.c_void_p)
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    pa = ctypes.cast(arr, P)
    fn = L.indexshare_group_fwd_noalloc
    a = args()
    assert fn(ctypes.byref(a), 64, 0, pa, pa, pa, pa, None, 16, 1, 128, ctypes.c_float(0.1),
              FAKE, None) == bd.IX_ERR_INVALID
    assert fn(ctypes.byref(a), 64, 4, pa, pa, pa, pa, None, 16, 1, 128, ctypes.c_float(0.1),
              None, None) == bd.IX_ERR_INVALID
    assert fn(ctypes.byref(a), 64, 4, pa, pa, pa, pa, None, 16, 1, 96, ctypes.c_float(0.1),
              FAKE, None) == bd.IX_ERR_UNSUPPORTED
    big = args(T=4096, S_max=4096)
    assert bd.indexshare_workspace_bytes(big, 2048, 16, 1, 128) > bd.NOALLOC_SCRATCH_BYTES
    assert fn(ctypes.byref(big), 2048, 4, pa, pa, pa, pa, None, 16, 1, 128, ctypes.c_float(0.1),
              FAKE, None) == bd.IX_ERR_WORKSPACE
    assert "scratch" in bd.ix_last_error()
    # a decode step at 128K keys fits
    dec = args(B=128, T=1, S_max=131072)
    assert 0 < bd.indexshare_workspace_bytes(dec, 2048, 16, 1, 128) <= bd.NOALLOC_SCRATCH_BYTES
    empty = args(B=0)
    assert fn(ctypes.byref(empty), 64, 4, pa, pa, pa, pa, None, 16, 1, 128, ctypes.c_float(0.1),
              FAKE, None) == bd.IX_OK


def test_append_validation_codes():
    ok = dict(kn=FAKE, Kn=FAKE, Vn=FAKE, pos0=FAKE, B=2, T=1, S=64, d_I=128, H_kv=1, d=128,
              kc=FAKE, Kc=FAKE, Vc=FAKE)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return status_of(bd.ix_append_kv, a["kn"], a["Kn"], a["Vn"], a["pos0"], a["B"], a["T"],
                         a["S"], a["d_I"], a["H_kv"], a["d"], a["kc"], a["Kc"], a["Vc"])

    assert call(kc=0) == bd.IX_ERR_INVALID            # new keys without a cache
    assert call(Kn=0) == bd.IX_ERR_INVALID            # K cache without new rows
    assert call(pos0=0) == bd.IX_ERR_INVALID
    assert call(B=-1) == bd.IX_ERR_INVALID
    assert call(kn=FAKE + 4) == bd.IX_ERR_INVALID     # fp32 rows must be 16-byte aligned
    assert call(kc=FAKE + 4) == bd.IX_ERR_INVALID     # FP8 cache rows 8-byte aligned
    assert call(d_I=96) == bd.IX_ERR_UNSUPPORTED
    assert call(d=80) == bd.IX_ERR_UNSUPPORTED
    assert call(H_kv=0) == bd.IX_ERR_UNSUPPORTED
    # empty calls launch nothing
    assert call(B=0) == bd.IX_OK and call(T=0) == bd.IX_OK
    assert call(kn=0, kc=0, Kn=0, Kc=0, Vn=0, Vc=0) == bd.IX_OK


def test_one_launch_row_limits():
    # a launch counts its work-items in 32 bits: at most 2^24 - 1 rows of 256-thread blocks
    top = (1 << 24) - 1
    assert bd.ix_topk_workspace_bytes(args(T=top), 64) > 0
    assert bd.ix_topk_workspace_bytes(args(T=top + 1), 64) == 0
    assert bd.ix_topk_workspace_bytes(args(B=1 << 12, T=1 << 12), 64) == 0
    assert status_of(bd.ix_topk, args(B=1 << 12, T=1 << 12), 64, FAKE, 0, FAKE, 1 << 30) == \
        bd.IX_ERR_UNSUPPORTED
    assert "one launch" in bd.ix_last_error()
    assert status_of(bd.ix_score, args(T=top + 1), 0, 4, FAKE) == bd.IX_ERR_UNSUPPORTED
    # attention rows count KV heads too
    assert bd.sparse_attn_bwd_workspace_bytes(1, top // 4, 128, 4, 128, 64, 1024) > 0
    assert bd.sparse_attn_bwd_workspace_bytes(1, (top + 1) // 4, 128, 4, 128, 64, 1024) == 0
    assert status_of(bd.sparse_attn_fwd, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 22, 1, 128, 16, 4,
                     128, 64, 0.1, FAKE, 0, 0, 0) == bd.IX_ERR_UNSUPPORTED
    # the append's rows, the pooled expansion's entries and the block-key pieces
    assert status_of(bd.ix_append_kv, FAKE, FAKE, FAKE, FAKE, 1 << 12, 1 << 12, 64, 128, 1, 128,
                     FAKE, FAKE, FAKE) == bd.IX_ERR_UNSUPPORTED
    fits = args(T=1 << 20, S_max=1 << 16)
    assert bd.ix_topk_pooled_workspace_bytes(fits, 16, 255) > 0
    assert bd.ix_topk_pooled_workspace_bytes(fits, 16, 256) == 0
    assert status_of(bd.ix_topk_pooled, fits, 16, 256, FAKE, FAKE, 1 << 40) == \
        bd.IX_ERR_UNSUPPORTED
    assert status_of(bd.ix_pool_keys, FAKE, FAKE, 1 << 8, 1 << 21, 128, 1, FAKE) == \
        bd.IX_ERR_UNSUPPORTED


def test_indexer_kl_validation_codes():
    ok = dict(q=FAKE, kc=FAKE, idx=FAKE, kvl=FAKE, lse=FAKE, sc=FAKE, B=2, T=3, S=64, H_q=16,
              H_kv=1, d=128, k=16, scale=0.1, loss=FAKE, dsc=FAKE)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return status_of(bd.ix_indexer_kl, a["q"], a["kc"], a["idx"], a["kvl"], a["lse"], a["sc"],
                         a["B"], a["T"], a["S"], a["H_q"], a["H_kv"], a["d"], a["k"], a["scale"],
                         a["loss"], a["dsc"])

    for name in ("q", "kc", "idx", "lse", "sc", "loss", "dsc"):
        assert call(**{name: 0}) == bd.IX_ERR_INVALID, name
    assert call(q=FAKE + 2) == bd.IX_ERR_INVALID
    assert call(scale=float("nan")) == bd.IX_ERR_INVALID
    assert call(k=4096) == bd.IX_ERR_UNSUPPORTED
    assert call(d=96) == bd.IX_ERR_UNSUPPORTED
    assert call(H_q=12, H_kv=8) == bd.IX_ERR_UNSUPPORTED
    assert call(B=0) == bd.IX_OK and call(T=0, q=0) == bd.IX_OK


def test_attention_bwd_validation_codes():
    ok = dict(q=FAKE, kc=FAKE, vc=FAKE, idx=FAKE, kvl=FAKE, out=FAKE, lse=FAKE, dout=FAKE, B=2,
              T=3, S=64, H_q=16, H_kv=1, d=128, k=16, scale=0.1, dq=FAKE, dk=FAKE, dv=FAKE,
              pr=bd.PAIR_ROWS_BF16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return status_of(bd.sparse_attn_bwd, a["q"], a["kc"], a["vc"], a["idx"], a["kvl"], a["out"],
                         a["lse"], a["dout"], a["B"], a["T"], a["S"], a["H_q"], a["H_kv"], a["d"],
                         a["k"], a["scale"], a["dq"], a["dk"], a["dv"], a["pr"])

    for name in ("q", "kc", "vc", "idx", "out", "lse", "dout", "dq", "dk", "dv"):
        assert call(**{name: 0}) == bd.IX_ERR_INVALID, name
    for name in ("q", "kc", "vc", "out", "dout"):
        assert call(**{name: FAKE + 4}) == bd.IX_ERR_INVALID, name      # bf16: 16-byte aligned
    for name in ("lse", "dq", "dk", "dv"):
        assert call(**{name: FAKE + 2}) == bd.IX_ERR_INVALID, name      # fp32: 4-byte aligned
    assert call(scale=float("inf")) == bd.IX_ERR_INVALID
    assert call(k=0) == bd.IX_ERR_UNSUPPORTED and call(d=96) == bd.IX_ERR_UNSUPPORTED
    assert call(H_q=12, H_kv=8) == bd.IX_ERR_UNSUPPORTED
    assert call(B=0, q=0, kc=0, vc=0, idx=0, out=0, lse=0, dout=0, dq=0, dk=0, dv=0) == bd.IX_OK
    # the pair-row precision is checked with or without a workspace
    for bad in (-1, 2):
        assert call(pr=bad) == bd.IX_ERR_INVALID
        assert "pair_rows" in bd.ix_last_error()
    # the atomic-free form's workspace
    names = ("q", "kc", "vc", "idx", "kvl", "out", "lse", "dout", "B", "T", "S", "H_q", "H_kv", "d",
             "k", "scale", "dq", "dk", "dv", "pr")
    a = [ok[n] for n in names]
    one = bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 128, 16, 1)
    six = bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 128, 16, 6)
    assert 0 < one < six
    assert bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 128, 16, 100) == six   # clamped to B*T
    assert bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 96, 16, 1) == 0
    assert bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 128, 16, 0) == 0
    assert status_of(bd.sparse_attn_bwd, *a, FAKE, one - 1) == bd.IX_ERR_WORKSPACE
    assert status_of(bd.sparse_attn_bwd, *a, 0, one) == bd.IX_ERR_WORKSPACE
    assert status_of(bd.sparse_attn_bwd, *a, FAKE + 8, one) == bd.IX_ERR_INVALID
    # fp32 pair rows: 1024 instead of 512 bytes per pair at d = 128 (6 rows of 16 pairs)
    one32 = bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 128, 16, 1, bd.PAIR_ROWS_FP32)
    six32 = bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 128, 16, 6, bd.PAIR_ROWS_FP32)
    assert six32 - six >= 6 * 16 * 512 and one32 > one
    assert bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 128, 16, 1, 2) == 0
    a32 = [dict(ok, pr=bd.PAIR_ROWS_FP32)[n] for n in names]
    assert status_of(bd.sparse_attn_bwd, *a32, FAKE, one) == bd.IX_ERR_WORKSPACE


def test_group_bwd_validation_codes():
    n = 2
    arr = [FAKE] * n
    ok = dict(idx=FAKE, kvl=FAKE, n=n, q=arr, kc=arr, vc=arr, out=arr, lse=arr, dout=arr, B=2, T=3,
              S=64, H_q=16, H_kv=1, d=128, k=16, scale=0.1, dq=arr, dk=arr, dv=arr)
    one = bd.sparse_attn_bwd_workspace_bytes(2, 3, 64, 1, 128, 16, 1)

    def call(ws=FAKE, nb=one, pr=bd.PAIR_ROWS_BF16, **kw):
        a = dict(ok)
        a.update(kw)
        return status_of(bd.indexshare_group_bwd, a["idx"], a["kvl"], a["n"], a["q"], a["kc"], a["vc"],
                         a["out"], a["lse"], a["dout"], a["B"], a["T"], a["S"], a["H_q"], a["H_kv"],
                         a["d"], a["k"], a["scale"], a["dq"], a["dk"], a["dv"], pr, ws, nb)

    assert call(n=0) == bd.IX_ERR_INVALID
    for name in ("q", "kc", "vc", "out", "lse", "dout", "dq", "dk", "dv"):
        assert call(**{name: None}) == bd.IX_ERR_INVALID, name
        assert call(**{name: [FAKE, 0]}) == bd.IX_ERR_INVALID, name
    assert call(idx=0) == bd.IX_ERR_INVALID
    assert call(dk=[FAKE, FAKE + 2]) == bd.IX_ERR_INVALID
    assert call(ws=0, nb=0) == bd.IX_ERR_WORKSPACE
    assert call(nb=one - 1) == bd.IX_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == bd.IX_ERR_INVALID
    assert call(d=96) == bd.IX_ERR_UNSUPPORTED
    assert call(pr=3) == bd.IX_ERR_INVALID
    assert call(pr=bd.PAIR_ROWS_FP32) == bd.IX_ERR_WORKSPACE    # a bf16-sized workspace
    assert call(B=0, ws=0, nb=0) == bd.IX_OK


def test_indexer_bwd_validation_codes():
    def call(a=None, k=16, idx=FAKE, ds=FAKE, dq=FAKE, dw=FAKE, dk=FAKE):
        return status_of(bd.ix_indexer_bwd, a if a is not None else args(), k, idx, ds, dq, dw, dk)

    for name in ("idx", "ds", "dq", "dw", "dk"):
        assert call(**{name: 0}) == bd.IX_ERR_INVALID, name
    assert "NULL" in bd.ix_last_error()
    assert call(a=args(w=0)) == bd.IX_ERR_INVALID
    for name in ("idx", "ds", "dq", "dw", "dk"):
        assert call(**{name: FAKE + 2}) == bd.IX_ERR_INVALID, name
    assert call(a=args(w=FAKE + 2)) == bd.IX_ERR_INVALID
    assert call(a=args(q=FAKE + 8)) == bd.IX_ERR_INVALID
    assert call(a=args(d_I=96)) == bd.IX_ERR_UNSUPPORTED
    assert call(a=args(H_I=6)) == bd.IX_ERR_UNSUPPORTED
    assert call(k=0) == bd.IX_ERR_UNSUPPORTED and call(k=4096) == bd.IX_ERR_UNSUPPORTED
    assert bd.load().ix_indexer_bwd(None, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, 0, None) == bd.IX_ERR_INVALID
    assert status_of(bd.ix_indexer_bwd, args(), 16, FAKE, FAKE, FAKE, FAKE, FAKE, 2) == bd.IX_ERR_INVALID
    assert "pair_rows" in bd.ix_last_error()
    # empty calls launch nothing
    assert call(a=args(B=0, q=0, k=0, w=0, q_pos0=0, kv_len=0), idx=0, ds=0, dq=0, dw=0, dk=0) == bd.IX_OK
    # the atomic-free form's workspace
    one = bd.ix_indexer_bwd_workspace_bytes(args(), 16, 1)
    assert 0 < one < bd.ix_indexer_bwd_workspace_bytes(args(), 16, 7)
    assert bd.ix_indexer_bwd_workspace_bytes(args(), 16, 10 ** 6) == \
        bd.ix_indexer_bwd_workspace_bytes(args(), 16, 128)                      # clamped to B*T
    assert bd.ix_indexer_bwd_workspace_bytes(args(d_I=96), 16, 1) == 0
    assert bd.ix_indexer_bwd_workspace_bytes(args(), 16, 1, -1) == 0
    a = args()
    bf, f32 = bd.PAIR_ROWS_BF16, bd.PAIR_ROWS_FP32
    assert status_of(bd.ix_indexer_bwd, a, 16, FAKE, FAKE, FAKE, FAKE, FAKE, bf, FAKE, one - 1) == bd.IX_ERR_WORKSPACE
    assert status_of(bd.ix_indexer_bwd, a, 16, FAKE, FAKE, FAKE, FAKE, FAKE, bf, 0, one) == bd.IX_ERR_WORKSPACE
    assert status_of(bd.ix_indexer_bwd, a, 16, FAKE, FAKE, FAKE, FAKE, FAKE, bf, FAKE + 8, one) == bd.IX_ERR_INVALID
    # fp32 dk_I rows: 512 instead of 256 bytes per pair at d_I = 128
    one32 = bd.ix_indexer_bwd_workspace_bytes(args(), 16, 1, f32)
    assert one32 >= one + 16 * 256
    assert status_of(bd.ix_indexer_bwd, a, 16, FAKE, FAKE, FAKE, FAKE, FAKE, f32, FAKE, one) == bd.IX_ERR_WORKSPACE


def test_debug_status_validation():
    assert status_of(bd.ix_debug_enable, 2) == bd.IX_ERR_INVALID
    assert status_of(bd.ix_debug_enable, -1) == bd.IX_ERR_INVALID
    assert bd.load().ix_debug_read(None, 0, None) == bd.IX_ERR_INVALID
    assert "NULL" in bd.ix_last_error()
    assert status_of(bd.ix_debug_enable, 1) == bd.IX_OK
    assert status_of(bd.ix_debug_enable, 0) == bd.IX_OK
    assert ctypes.sizeof(bd.DebugStatus) == 5 * 8


def test_peak_validation_codes():
    assert status_of(pk.ix_peak_mfma_fp8, 0, 8, 1, 1, FAKE) == bd.IX_ERR_INVALID
    assert "NULL" in pk.load().ix_peak_last_error().decode()
    assert status_of(pk.ix_peak_mfma_fp8, FAKE, 6, 1, 1, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_mfma_fp8, FAKE, 8, 0, 1, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_copy, FAKE, FAKE, 24) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_copy, FAKE, FAKE, 0) == bd.IX_OK
    assert status_of(pk.ix_peak_read, FAKE, 24, 1024, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_read, 0, 32, 1024, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_read, FAKE, 32, 0, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_read, FAKE, 32, 65537, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_read, FAKE, 32, 1024, 2, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_read, FAKE, 0, 1024, 1, FAKE) == bd.IX_OK
    assert status_of(pk.ix_peak_gather, FAKE, 1000, FAKE, 5, 2048, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_gather, FAKE, 1 << 32, FAKE, 5, 2048, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_gather, FAKE, 256, FAKE, -1, 2048, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_gather, FAKE, 256, FAKE, 5, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_gather, FAKE, 256, FAKE, 0, 2048, FAKE) == bd.IX_OK
    wide = pk.ix_peak_gather_wide
    assert status_of(wide, FAKE, 1000, 2, FAKE, 5, 2048, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(wide, FAKE, (1 << 30) + 256, 2, FAKE, 5, 2048, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(wide, FAKE, 256, 0, FAKE, 5, 2048, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(wide, FAKE, 256, 65, FAKE, 5, 2048, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(wide, FAKE, 256, 2, FAKE, -1, 2048, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(wide, FAKE, 256, 2, FAKE, 5, 0, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(wide, FAKE, 256, 2, FAKE, 5, 2048, 2, FAKE) == bd.IX_ERR_INVALID
    assert status_of(wide, 0, 256, 2, FAKE, 5, 2048, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(wide, FAKE, 1 << 30, 64, FAKE, 0, 2048, 1, FAKE) == bd.IX_OK
    sel = pk.ix_peak_gather_selection
    assert status_of(sel, FAKE, FAKE, 0, FAKE, 1, 4, 100, 1, 128, 64, 1, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(sel, FAKE, FAKE, FAKE, FAKE, 1, 4, 100, 1, 96, 64, 1, 0, FAKE) == bd.IX_ERR_UNSUPPORTED
    assert status_of(sel, FAKE, FAKE, FAKE, FAKE, 1, 4, 100, 1, 128, 4096, 1, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(sel, FAKE, FAKE, FAKE, FAKE, 1, 4, 100, 1, 128, 64, 0, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(sel, FAKE, FAKE, FAKE, FAKE, 1, 4, 100, 1, 128, 64, 1, 1, FAKE) == bd.IX_ERR_INVALID
    assert status_of(sel, FAKE + 8, FAKE, FAKE, FAKE, 1, 4, 100, 1, 128, 64, 1, 0, FAKE) == bd.IX_ERR_INVALID
    assert status_of(sel, FAKE, FAKE, FAKE, FAKE, 0, 4, 100, 1, 128, 64, 1, 2, FAKE) == bd.IX_OK
    assert status_of(pk.ix_peak_atomic_add, 0, 10, FAKE, 5) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_atomic_add, FAKE, 0, FAKE, 5) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_atomic_add, FAKE, (1 << 24) + 1, FAKE, 5) == bd.IX_ERR_INVALID
    assert status_of(pk.ix_peak_atomic_add, FAKE, 10, FAKE, 0) == bd.IX_OK


def test_workspace_sizes_for_the_named_workloads():
    from indexed_sparse_attention_ix_amd.workloads import WORKLOADS
    for wl in WORKLOADS.values():
        a = args(B=wl.B, T=wl.T, S_max=wl.S, H_I=wl.H_I, d_I=wl.d_I)
        nb = bd.ix_topk_workspace_bytes(a, wl.k)
        assert 0 < nb < 16 << 30   # fits comfortably in 288 GB of HBM
        assert bd.indexshare_workspace_bytes(a, wl.k, wl.H_q, wl.H_kv, wl.d) >= nb
