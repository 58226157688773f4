"""IX_ERR_HIP without a GPU: in the test build of the library (-DIX_TEST_HOOKS, loaded through
IX_LIB by test_abi_sanitized.py) a hook makes every launch report a chosen HIP error before
anything is launched.  Each entry point, called with valid arguments, must then return
IX_ERR_HIP with a message naming the call and the HIP error.  The release library has no hook,
and there these tests are skipped (they would launch on stand-in pointers)."""
import ctypes

import pytest

from indexed_sparse_attention_ix_amd import binding as bd

FAKE = 1 << 20          # 16-byte aligned stand-in address: nothing is dereferenced
HIP_ERROR_LAUNCH_FAILURE = 719


def _hooked_lib():
    lib = ctypes.CDLL(bd.LIB_PATH)
    if not hasattr(lib, "ix_test_fail_launches"):
        pytest.skip("the release library has no launch hook")
    lib.ix_test_fail_launches.argtypes = [ctypes.c_int32]
    lib.ix_test_fail_launches.restype = None
    return lib


def _args(**kw):
    d = dict(B=2, T=16, S_max=256, H_I=64, d_I=128)
    d.update(kw)
    return bd.IndexerArgs(FAKE, FAKE, FAKE, FAKE, FAKE, d["B"], d["T"], d["S_max"], d["H_I"], d["d_I"])


def _calls():
    """One valid call of every entry point that launches (name, thunk returning a status)."""
    L = bd.load()
    P = ctypes.POINTER(ctypes.c_void_p)
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    pa = ctypes.cast(arr, P)
    fa = ctypes.cast((ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE), P)
    a = _args()
    ws_t = bd.ix_topk_workspace_bytes(a, 64)
    ws_g = bd.indexshare_workspace_bytes(a, 64, 16, 1, 128)
    ws_a = bd.sparse_attn_workspace_bytes(2, 16, 16, 1, 128, 64)
    ws_p = bd.ix_topk_pooled_workspace_bytes(a, 4, 16)
    sc = ctypes.c_float(0.1)
    attn = (FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, 256, 16, 1, 128, 64, sc)
    return [
        ("ix_score", lambda: L.ix_score(ctypes.byref(a), 0, 16, FAKE, None)),
        ("ix_topk", lambda: L.ix_topk(ctypes.byref(a), 64, FAKE, None, FAKE, ws_t, None)),
        ("sparse_attn_fwd", lambda: L.sparse_attn_fwd(*attn, FAKE, None, FAKE, max(ws_a, 16), None)),
        ("sparse_attn_group_fwd", lambda: L.sparse_attn_group_fwd(
            4, pa, pa, pa, pa, None, FAKE, FAKE, 2, 16, 256, 16, 1, 128, 64, sc, FAKE, 1 << 20, None)),
        ("indexshare_group_fwd", lambda: L.indexshare_group_fwd(
            ctypes.byref(a), 64, 4, pa, pa, pa, pa, None, 16, 1, 128, sc, FAKE, FAKE, ws_g, None)),
        ("indexshare_group_fwd_noalloc", lambda: L.indexshare_group_fwd_noalloc(
            ctypes.byref(a), 64, 4, pa, pa, pa, pa, None, 16, 1, 128, sc, FAKE, None)),
        ("ix_append_kv", lambda: L.ix_append_kv(FAKE, FAKE, FAKE, FAKE, 2, 1, 256, 128, 1, 128,
                                                FAKE, FAKE, FAKE, None)),
        ("ix_pool_keys", lambda: L.ix_pool_keys(FAKE, FAKE, 2, 256, 128, 4, FAKE, None)),
        ("ix_topk_pooled", lambda: L.ix_topk_pooled(ctypes.byref(a), 4, 16, FAKE, FAKE, ws_p, None)),
        ("sparse_attn_bwd", lambda: L.sparse_attn_bwd(
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, 256, 16, 1, 128, 64, sc, FAKE,
            FAKE, FAKE, bd.PAIR_ROWS_BF16, None, 0, None)),
        ("indexshare_group_bwd", lambda: L.indexshare_group_bwd(
            FAKE, FAKE, 4, pa, pa, pa, pa, fa, pa, 2, 16, 256, 16, 1, 128, 64, sc, fa, fa, fa,
            bd.PAIR_ROWS_FP32, FAKE,
            bd.sparse_attn_bwd_workspace_bytes(2, 16, 256, 1, 128, 64, 32, bd.PAIR_ROWS_FP32), None)),
        ("ix_indexer_kl", lambda: L.ix_indexer_kl(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, 256, 16,
                                                  1, 128, 64, sc, FAKE, FAKE, None)),
        ("ix_indexer_bwd", lambda: L.ix_indexer_bwd(ctypes.byref(a), 64, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                    bd.PAIR_ROWS_BF16, None, 0, None)),
        ("ix_debug_read", lambda: L.ix_debug_read(ctypes.byref(bd.DebugStatus()), 1, None)),
    ]


@pytest.mark.parametrize("debug", [0, 1])
def test_every_launching_entry_point_reports_the_hip_error(debug):
    """With the debug status on, the calls first look up its address or check idx: the
    failure of those steps is reported the same way."""
    lib = _hooked_lib()
    lib.ix_test_fail_launches(HIP_ERROR_LAUNCH_FAILURE)
    bd.ix_debug_enable(debug)
    try:
        for name, call in _calls():
            st = call()
            msg = bd.ix_last_error()
            assert st == bd.IX_ERR_HIP, f"{name}: status {st} ({msg})"
            assert any(w in msg for w in ("launch", "scratch", "debug")), f"{name}: {msg}"
            assert len(msg) > len(name), f"{name}: no HIP error text in {msg!r}"
    finally:
        lib.ix_test_fail_launches(0)
        bd.ix_debug_enable(0)
    # a failing validation still wins over the hook, and a clean status clears the message
    lib.ix_test_fail_launches(HIP_ERROR_LAUNCH_FAILURE)
    try:
        assert bd.load().ix_topk(None, 64, FAKE, None, FAKE, 1, None) == bd.IX_ERR_INVALID
        empty = _args(B=0)
        assert bd.load().ix_topk(ctypes.byref(empty), 64, 0, None, 0, 0, None) == bd.IX_OK
        assert bd.ix_last_error() == ""
    finally:
        lib.ix_test_fail_launches(0)
