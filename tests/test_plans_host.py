"""Invariants of the launch plans over many shapes, on the host: the test build of the library
(-DIX_TEST_HOOKS, loaded through IX_LIB by test_abi_sanitized.py) exports ix_test_attn_plan and
ix_test_topk_plan.  The release library has neither, and there these tests are skipped."""
import ctypes
import itertools
import math

import pytest

from indexed_sparse_attention_ix_amd import binding as bd

FAKE = 1 << 20  # 16-byte aligned stand-in address: the plans dereference nothing
ATTN_FIELDS = ("layers", "n_splits", "light", "chunks", "chunks_per_split", "part_bytes", "ws_bytes")
TOPK_FIELDS = ("qc", "hc", "g", "gmax", "qgroups", "n_splits", "split_len", "cap", "ksplit",
               "fb_cap", "samp_tiles", "fb_samp_tiles", "units", "ws_bytes")
WAVES = 4  # waves per attention block


def _lib():
    lib = ctypes.CDLL(bd.LIB_PATH)
    if not hasattr(lib, "ix_test_attn_plan"):
        pytest.skip("the release library has no plan hooks")
    lib.ix_test_attn_plan.restype = ctypes.c_int32
    lib.ix_test_attn_plan.argtypes = [ctypes.c_int32] * 7 + [ctypes.POINTER(ctypes.c_int64)]
    lib.ix_test_topk_plan.restype = ctypes.c_int32
    lib.ix_test_topk_plan.argtypes = [ctypes.POINTER(bd.IndexerArgs), ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64)]
    return lib


def _attn_plan(lib, B, T, H_q, H_kv, d, k, layers):
    out = (ctypes.c_int64 * 8)()
    n = lib.ix_test_attn_plan(B, T, H_q, H_kv, d, k, layers, out)
    return dict(zip(ATTN_FIELDS, out[:n]))


def _topk_plan(lib, a, k):
    out = (ctypes.c_int64 * 16)()
    n = lib.ix_test_topk_plan(ctypes.byref(a), k, out)
    return dict(zip(TOPK_FIELDS, out[:n]))


def test_attention_plans():
    """Every chunk of the selection belongs to a split, a split gives each wave at least two
    chunks, small grids (decode) take the light kernel and share launches, split towards one
    block per CU, large grids run one layer per launch unsplit with the main kernel, and the
    ABI's workspace sizes are the plan's."""
    lib = _lib()
    n = 0
    for B, T, H_kv, d, k, layers in itertools.product((1, 2, 64), (1, 3, 150, 600, 4096),
                                                      (1, 2), (64, 128), (1, 37, 256, 2048),
                                                      (1, 2, 4, 8, 9)):
        H_q = 8 * H_kv
        p = _attn_plan(lib, B, T, H_q, H_kv, d, k, layers)
        base = B * T * H_kv
        where = f"B={B} T={T} H_kv={H_kv} d={d} k={k} layers={layers}: {p}"
        chunk = 16 if p["light"] else 32
        assert p["chunks"] == math.ceil(k / chunk), where
        assert p["n_splits"] >= 1 and p["chunks_per_split"] * p["n_splits"] >= p["chunks"], where
        if p["n_splits"] > 1:
            assert p["chunks_per_split"] >= 2 * WAVES, where
            need = base * p["n_splits"] * 16 * (d + 1) * 4
            assert p["part_bytes"] >= need, where
        else:
            assert p["part_bytes"] == 0, where
        if base >= 1024:
            assert p["layers"] == 1 and p["n_splits"] == 1 and not p["light"], where
        else:
            assert p["layers"] == min(layers, 8) and p["light"], where
            blocks = base * p["layers"] * p["n_splits"]
            if p["n_splits"] > 1:
                assert blocks <= 256 + base * p["layers"] // 2 + base * p["layers"], where
            if p["chunks"] >= 2 * WAVES * 2 and base * p["layers"] <= 128:
                assert p["n_splits"] > 1, where  # a small launch is split
        assert base * p["n_splits"] * p["layers"] < 2 ** 31, where
        assert p["ws_bytes"] == p["layers"] * p["part_bytes"], where
        if layers == 1:
            assert bd.sparse_attn_workspace_bytes(B, T, H_q, H_kv, d, k) == p["ws_bytes"], where
        assert bd.sparse_attn_group_workspace_bytes(B, T, H_q, H_kv, d, k, layers) == p["ws_bytes"], where
        n += 1
    assert n > 500


def _stage(gmax):
    """Entries of a wave's LDS stage: two blocks of appends per key tile in flight (2 tiles in
    flight with 16 head blocks of operands, 4 with 8, 8 with fewer)."""
    pf = 2 if gmax >= 16 else 4 if gmax >= 8 else 8
    return 2 * 64 * pf


def test_topk_plans():
    """The wave units cover every query and key once, a split keeps at most k entries, a
    candidate buffer holds k' entries, a full stage and the slack between compactions, a
    threshold sample fits a buffer without a compaction, and the ABI's workspace size is the
    plan's."""
    lib = _lib()
    n = 0
    for B, T, S, H_I, d_I, k in itertools.product((1, 2, 64), (1, 2, 3, 4, 5, 150, 4096),
                                                  (17, 1000, 4096, 131072, 1048576),
                                                  (4, 16, 20, 64), (64, 128), (1, 37, 256, 2048)):
        a = bd.IndexerArgs(FAKE, FAKE, FAKE, FAKE, FAKE, B, T, S, H_I, d_I)
        ws = bd.ix_topk_workspace_bytes(a, k)
        if ws == 0:
            continue  # outside the supported shapes
        p = _topk_plan(lib, a, k)
        where = f"B={B} T={T} S={S} H_I={H_I} d_I={d_I} k={k}: {p}"
        assert p["qc"] == (1 if T < 4 and H_I % 16 == 0 else 4), where
        assert p["hc"] * p["qc"] == 16 and p["g"] * p["hc"] == H_I, where
        assert p["gmax"] in (1, 2, 4, 8, 16) and p["g"] <= p["gmax"] < 2 * max(p["g"], 1), where
        assert p["qgroups"] == math.ceil(T / p["qc"]), where
        ns = p["n_splits"]
        assert 1 <= ns <= 64 and p["split_len"] % 16 == 0, where
        assert p["split_len"] * ns >= S and (ns - 1) * p["split_len"] < S, where
        assert p["units"] == B * p["qgroups"] * ns, where
        assert p["ksplit"] <= k and (ns > 1 or p["ksplit"] == k), where
        stage = _stage(p["gmax"])
        pad = lambda x: math.ceil(x / 64) * 64
        assert p["cap"] >= 2 * pad(p["ksplit"]) + 2 * stage, where
        assert p["fb_cap"] >= 2 * pad(k) + 2 * stage, where
        assert p["samp_tiles"] * 16 + stage <= p["cap"], where
        assert p["fb_samp_tiles"] * 16 + stage <= p["fb_cap"], where
        assert p["ws_bytes"] == ws, where
        assert ws >= B * T * ns * p["cap"] * 8, where
        n += 1
    assert n > 1000
