"""ctypes binding of libix.so: the C ABI of include/ix.h with the same entry-point names.

Two layers, both argument marshalling only:
  * raw functions (`ix_score`, `ix_topk`, `sparse_attn_fwd`, `indexshare_group_fwd`,
    the `*_workspace_bytes` queries, `ix_last_error`) take device pointers as ints and
    a HIP stream handle, exactly like the C functions, and raise IxError on a non-OK
    status;
  * tensor helpers (`score`, `topk`, `sparse_attention`, `indexshare_group`) take torch
    device tensors, allocate outputs and workspaces with torch (device memory is
    plumbing) and launch on torch's current stream.
Every step of the computation runs in the HIP kernels; there is no other code path.
If the library is not built (or cannot be loaded) every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional, Sequence

# IX_LIB names another build of the same ABI (the CPU tests load a sanitized host-only one).
LIB_PATH = os.environ.get("IX_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                    "libix.so")

ABI_VERSION = 5  # IX_ABI_VERSION of include/ix.h
IX_OK, IX_ERR_INVALID, IX_ERR_UNSUPPORTED, IX_ERR_WORKSPACE, IX_ERR_HIP = 0, -1, -2, -3, -4
PAIR_ROWS_BF16, PAIR_ROWS_FP32 = 0, 1  # ix_pair_rows of include/ix.h
STATUS_NAMES = {0: "IX_OK", -1: "IX_ERR_INVALID", -2: "IX_ERR_UNSUPPORTED",
                -3: "IX_ERR_WORKSPACE", -4: "IX_ERR_HIP"}

# every symbol include/ix.h declares
EXPORTS = ("ix_abi_version", "ix_last_error", "ix_score", "ix_topk_workspace_bytes", "ix_topk",
           "sparse_attn_workspace_bytes", "sparse_attn_fwd", "sparse_attn_group_workspace_bytes",
           "sparse_attn_group_fwd", "indexshare_workspace_bytes",
           "indexshare_group_fwd", "indexshare_group_fwd_noalloc", "ix_append_kv",
           "ix_pool_keys", "ix_topk_pooled_workspace_bytes", "ix_topk_pooled", "sparse_attn_bwd",
           "sparse_attn_bwd_workspace_bytes", "indexshare_group_bwd", "ix_indexer_kl",
           "ix_indexer_bwd", "ix_indexer_bwd_workspace_bytes", "ix_debug_enable", "ix_debug_read")


class IxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class IndexerArgs(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("k", c_void_p), ("w", c_void_p), ("q_pos0", c_void_p),
                ("kv_len", c_void_p), ("B", c_int32), ("T", c_int32), ("S_max", c_int32),
                ("H_I", c_int32), ("d_I", c_int32)]


class DebugStatus(ctypes.Structure):
    """ix_debug_status of include/ix.h."""
    _fields_ = [("idx_out_of_range", ctypes.c_uint64), ("topk_compactions", ctypes.c_uint64),
                ("topk_resweeps", ctypes.c_uint64), ("topk_split_recomputes", ctypes.c_uint64),
                ("topk_overflow", ctypes.c_uint64)]


_lib = None


def load(path: str = LIB_PATH):
    """Loads libix.so (once) and declares the prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libix.so not built at {path}; run __graft_entry__.build() or "
                           f"python -m indexed_sparse_attention_ix_amd.build")
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    L.ix_abi_version.restype = c_int32
    L.ix_abi_version.argtypes = []
    L.ix_last_error.restype = ctypes.c_char_p
    L.ix_last_error.argtypes = []
    L.ix_score.restype = c_int32
    L.ix_score.argtypes = [P(IndexerArgs), c_int32, c_int32, c_void_p, c_void_p]
    L.ix_topk_workspace_bytes.restype = c_size_t
    L.ix_topk_workspace_bytes.argtypes = [P(IndexerArgs), c_int32]
    L.ix_topk.restype = c_int32
    L.ix_topk.argtypes = [P(IndexerArgs), c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                          c_void_p]
    L.sparse_attn_workspace_bytes.restype = c_size_t
    L.sparse_attn_workspace_bytes.argtypes = [c_int32] * 6
    L.sparse_attn_fwd.restype = c_int32
    L.sparse_attn_fwd.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                  c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    L.sparse_attn_group_workspace_bytes.restype = c_size_t
    L.sparse_attn_group_workspace_bytes.argtypes = [c_int32] * 7
    L.sparse_attn_group_fwd.restype = c_int32
    L.sparse_attn_group_fwd.argtypes = ([c_int32] + [P(c_void_p)] * 5 + [c_void_p, c_void_p] +
                                        [c_int32] * 7 + [c_float, c_void_p, c_size_t, c_void_p])
    L.indexshare_workspace_bytes.restype = c_size_t
    L.indexshare_workspace_bytes.argtypes = [P(IndexerArgs), c_int32, c_int32, c_int32, c_int32]
    L.indexshare_group_fwd.restype = c_int32
    L.indexshare_group_fwd.argtypes = [P(IndexerArgs), c_int32, c_int32, P(c_void_p),
                                       P(c_void_p), P(c_void_p), P(c_void_p), P(c_void_p),
                                       c_int32, c_int32, c_int32, c_float, c_void_p, c_void_p,
                                       c_size_t, c_void_p]
    L.indexshare_group_fwd_noalloc.restype = c_int32
    L.indexshare_group_fwd_noalloc.argtypes = [P(IndexerArgs), c_int32, c_int32, P(c_void_p),
                                               P(c_void_p), P(c_void_p), P(c_void_p),
                                               P(c_void_p), c_int32, c_int32, c_int32, c_float,
                                               c_void_p, c_void_p]
    L.sparse_attn_bwd.restype = c_int32
    L.sparse_attn_bwd.argtypes = ([c_void_p] * 8 + [c_int32] * 7 + [c_float] + [c_void_p] * 3 +
                                  [c_int32, c_void_p, c_size_t, c_void_p])
    L.indexshare_group_bwd.restype = c_int32
    L.indexshare_group_bwd.argtypes = ([c_void_p, c_void_p, c_int32] + [P(c_void_p)] * 6 +
                                       [c_int32] * 7 + [c_float] + [P(c_void_p)] * 3 +
                                       [c_int32, c_void_p, c_size_t, c_void_p])
    L.sparse_attn_bwd_workspace_bytes.restype = c_size_t
    L.sparse_attn_bwd_workspace_bytes.argtypes = [c_int32] * 8
    L.ix_indexer_bwd.restype = c_int32
    L.ix_indexer_bwd.argtypes = ([P(IndexerArgs), c_int32] + [c_void_p] * 5 +
                                 [c_int32, c_void_p, c_size_t, c_void_p])
    L.ix_indexer_bwd_workspace_bytes.restype = c_size_t
    L.ix_indexer_bwd_workspace_bytes.argtypes = [P(IndexerArgs), c_int32, c_int32, c_int32]
    L.ix_indexer_kl.restype = c_int32
    L.ix_indexer_kl.argtypes = [c_void_p] * 6 + [c_int32] * 7 + [c_float] + [c_void_p] * 3
    L.ix_pool_keys.restype = c_int32
    L.ix_pool_keys.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                               c_void_p]
    L.ix_topk_pooled_workspace_bytes.restype = c_size_t
    L.ix_topk_pooled_workspace_bytes.argtypes = [P(IndexerArgs), c_int32, c_int32]
    L.ix_topk_pooled.restype = c_int32
    L.ix_topk_pooled.argtypes = [P(IndexerArgs), c_int32, c_int32, c_void_p, c_void_p, c_size_t,
                                 c_void_p]
    L.ix_append_kv.restype = c_int32
    L.ix_append_kv.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                               c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
    L.ix_debug_enable.restype = c_int32
    L.ix_debug_enable.argtypes = [c_int32]
    L.ix_debug_read.restype = c_int32
    L.ix_debug_read.argtypes = [P(DebugStatus), c_int32, c_void_p]
    if L.ix_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {L.ix_abi_version()}, this binding expects "
                           f"{ABI_VERSION}: rebuild with __graft_entry__.build()")
    _lib = L
    return L


def _check(status: int):
    if status != IX_OK:
        raise IxError(status, load().ix_last_error().decode(errors="replace"))


# ------------------------------------------------------------------ raw C-ABI mirrors


def ix_abi_version() -> int:
    return load().ix_abi_version()


def ix_last_error() -> str:
    return load().ix_last_error().decode(errors="replace")


def ix_score(args: IndexerArgs, t_begin: int, t_end: int, scores: int, stream: int = 0):
    _check(load().ix_score(ctypes.byref(args), t_begin, t_end, scores, stream))


def ix_topk_workspace_bytes(args: IndexerArgs, k: int) -> int:
    return load().ix_topk_workspace_bytes(ctypes.byref(args), k)


def ix_topk(args: IndexerArgs, k: int, idx: int, sel_scores: int, ws: int, ws_bytes: int,
            stream: int = 0):
    _check(load().ix_topk(ctypes.byref(args), k, idx, sel_scores, ws, ws_bytes, stream))


def sparse_attn_workspace_bytes(B, T, H_q, H_kv, d, k) -> int:
    return load().sparse_attn_workspace_bytes(B, T, H_q, H_kv, d, k)


def sparse_attn_fwd(q, kc, vc, idx, kv_len, B, T, S_max, H_q, H_kv, d, k, sm_scale, out, lse,
                    ws, ws_bytes, stream=0):
    _check(load().sparse_attn_fwd(q, kc, vc, idx, kv_len, B, T, S_max, H_q, H_kv, d, k,
                                  sm_scale, out, lse, ws, ws_bytes, stream))


def sparse_attn_group_workspace_bytes(B, T, H_q, H_kv, d, k, n_layers) -> int:
    return load().sparse_attn_group_workspace_bytes(B, T, H_q, H_kv, d, k, n_layers)


def sparse_attn_group_fwd(n_layers, q, kc, vc, out, lse, idx, kv_len, B, T, S_max, H_q, H_kv, d,
                          k, sm_scale, ws, ws_bytes, stream=0):
    keep = []
    conv = []
    for ptrs in (q, kc, vc, out, lse):
        r = _ptr_array(ptrs)
        if r is None:
            conv.append(None)
        else:
            conv.append(r[0])
            keep.append(r[1])
    _check(load().sparse_attn_group_fwd(n_layers, *conv, idx, kv_len, B, T, S_max, H_q, H_kv, d,
                                        k, sm_scale, ws, ws_bytes, stream))


def indexshare_workspace_bytes(args: IndexerArgs, k, H_q, H_kv, d) -> int:
    return load().indexshare_workspace_bytes(ctypes.byref(args), k, H_q, H_kv, d)


def _ptr_array(ptrs: Optional[Sequence[int]]):
    if ptrs is None:
        return None
    arr = (c_void_p * len(ptrs))(*[p if p else None for p in ptrs])
    return ctypes.cast(arr, ctypes.POINTER(c_void_p)), arr


def indexshare_group_fwd(args: IndexerArgs, k, n_layers, q, kc, vc, out, lse, H_q, H_kv, d,
                         sm_scale, idx, ws, ws_bytes, stream=0):
    keep = []
    conv = []
    for ptrs in (q, kc, vc, out, lse):
        r = _ptr_array(ptrs)
        if r is None:
            conv.append(None)
        else:
            conv.append(r[0])
            keep.append(r[1])
    _check(load().indexshare_group_fwd(ctypes.byref(args), k, n_layers, conv[0], conv[1],
                                       conv[2], conv[3], conv[4], H_q, H_kv, d, sm_scale, idx,
                                       ws, ws_bytes, stream))


NOALLOC_SCRATCH_BYTES = 64 << 20  # IX_NOALLOC_SCRATCH_BYTES of include/ix.h


def indexshare_group_fwd_noalloc(args: IndexerArgs, k, n_layers, q, kc, vc, out, lse, H_q, H_kv,
                                 d, sm_scale, idx, stream=0):
    keep = []
    conv = []
    for ptrs in (q, kc, vc, out, lse):
        r = _ptr_array(ptrs)
        if r is None:
            conv.append(None)
        else:
            conv.append(r[0])
            keep.append(r[1])
    _check(load().indexshare_group_fwd_noalloc(ctypes.byref(args), k, n_layers, conv[0], conv[1],
                                               conv[2], conv[3], conv[4], H_q, H_kv, d, sm_scale,
                                               idx, stream))


def ix_append_kv(k_I_new, K_new, V_new, pos0, B, T_new, S_max, d_I, H_kv, d, k_I_cache,
                 K_cache, V_cache, stream=0):
    _check(load().ix_append_kv(k_I_new, K_new, V_new, pos0, B, T_new, S_max, d_I, H_kv, d,
                               k_I_cache, K_cache, V_cache, stream))


def ix_debug_enable(on: int):
    _check(load().ix_debug_enable(on))


def ix_debug_read(reset: int = 0, stream: int = 0) -> dict:
    """The debug status of the stream's GPU (ix_debug_read) as a dict of its counters."""
    st = DebugStatus()
    _check(load().ix_debug_read(ctypes.byref(st), reset, stream))
    return {name: int(getattr(st, name)) for name, _ in DebugStatus._fields_}


def sparse_attn_bwd(q, kc, vc, idx, kv_len, out, lse, dout, B, T, S_max, H_q, H_kv, d, k,
                    sm_scale, dq, dkc, dvc, pair_rows=0, ws=0, ws_bytes=0, stream=0):
    _check(load().sparse_attn_bwd(q, kc, vc, idx, kv_len, out, lse, dout, B, T, S_max, H_q,
                                  H_kv, d, k, sm_scale, dq, dkc, dvc, pair_rows, ws, ws_bytes,
                                  stream))


def indexshare_group_bwd(idx, kv_len, n_layers, q, kc, vc, out, lse, dout, B, T, S_max, H_q,
                         H_kv, d, k, sm_scale, dq, dkc, dvc, pair_rows, ws, ws_bytes, stream=0):
    keep = []
    conv = []
    for ptrs in (q, kc, vc, out, lse, dout, dq, dkc, dvc):
        r = _ptr_array(ptrs)
        conv.append(None if r is None else r[0])
        if r is not None:
            keep.append(r[1])
    _check(load().indexshare_group_bwd(idx, kv_len, n_layers, *conv[:6], B, T, S_max, H_q, H_kv,
                                       d, k, sm_scale, *conv[6:], pair_rows, ws, ws_bytes,
                                       stream))


def sparse_attn_bwd_workspace_bytes(B, T, S_max, H_kv, d, k, rows_per_pass, pair_rows=0):
    return load().sparse_attn_bwd_workspace_bytes(B, T, S_max, H_kv, d, k, rows_per_pass,
                                                  pair_rows)






def ix_indexer_kl(q, kc, idx, kv_len, lse, sel_scores, B, T, S_max, H_q, H_kv, d, k, sm_scale,
                  loss, dscores, stream=0):
    _check(load().ix_indexer_kl(q, kc, idx, kv_len, lse, sel_scores, B, T, S_max, H_q, H_kv, d,
                                k, sm_scale, loss, dscores, stream))


def ix_pool_keys(k_I, kv_len, B, S_max, d_I, pool, k_pooled, stream=0):
    _check(load().ix_pool_keys(k_I, kv_len, B, S_max, d_I, pool, k_pooled, stream))


def ix_topk_pooled_workspace_bytes(args: IndexerArgs, pool: int, k_blocks: int) -> int:
    return load().ix_topk_pooled_workspace_bytes(ctypes.byref(args), pool, k_blocks)


def ix_topk_pooled(args: IndexerArgs, pool, k_blocks, idx, ws, ws_bytes, stream=0):
    _check(load().ix_topk_pooled(ctypes.byref(args), pool, k_blocks, idx, ws, ws_bytes, stream))


# ------------------------------------------------------------------ torch tensor helpers


def _torch():
    import torch
    return torch


def _stream() -> int:
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def indexer_args(q_I, k_I, w, q_pos0, kv_len) -> IndexerArgs:
    """Builds the C struct from device tensors q_I [B,T,H_I,d_I] u8, k_I [B,S,d_I] u8,
    w [B,T,H_I] f32, q_pos0 [B] i32, kv_len [B] i32 (all contiguous)."""
    B, T, H, D = q_I.shape
    S = k_I.shape[1]
    for t in (q_I, k_I, w, q_pos0, kv_len):
        assert t.is_contiguous(), "indexer tensors must be contiguous"
    return IndexerArgs(_ptr(q_I), _ptr(k_I), _ptr(w), _ptr(q_pos0), _ptr(kv_len), B, T, S, H, D)


def workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def score(q_I, k_I, w, q_pos0, kv_len, t_begin=0, t_end=None):
    """fp32 scores [B, t_end - t_begin, S_max] (-inf where not visible)."""
    torch = _torch()
    a = indexer_args(q_I, k_I, w, q_pos0, kv_len)
    t_end = a.T if t_end is None else t_end
    out = torch.empty((a.B, t_end - t_begin, a.S_max), dtype=torch.float32, device=q_I.device)
    ix_score(a, t_begin, t_end, _ptr(out), _stream())
    return out


def topk(q_I, k_I, w, q_pos0, kv_len, k, with_scores=False, ws=None):
    """idx int32 [B,T,k] (ascending, -1 padded) and optionally the kept scores."""
    torch = _torch()
    a = indexer_args(q_I, k_I, w, q_pos0, kv_len)
    idx = torch.empty((a.B, a.T, k), dtype=torch.int32, device=q_I.device)
    sel = torch.empty((a.B, a.T, k), dtype=torch.float32, device=q_I.device) if with_scores else None
    nb = ix_topk_workspace_bytes(a, k)
    if ws is None or ws.numel() < nb:
        ws = workspace(nb, q_I.device)
    ix_topk(a, k, _ptr(idx), _ptr(sel), _ptr(ws), ws.numel(), _stream())
    return (idx, sel) if with_scores else idx


def sparse_attention(q, K, V, idx, sm_scale, kv_len=None, with_lse=False, ws=None):
    """bf16 out [B,T,H_q,d] (and fp32 lse [B,T,H_q]) over the selected rows."""
    torch = _torch()
    B, T, H_q, d = q.shape
    S, H_kv = K.shape[1], K.shape[2]
    k = idx.shape[2]
    for t in (q, K, V, idx):
        assert t.is_contiguous(), "attention tensors must be contiguous"
    out = torch.empty_like(q)
    lse = torch.empty((B, T, H_q), dtype=torch.float32, device=q.device) if with_lse else None
    nb = sparse_attn_workspace_bytes(B, T, H_q, H_kv, d, k)
    if nb and (ws is None or ws.numel() < nb):
        ws = workspace(nb, q.device)
    sparse_attn_fwd(_ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(kv_len), B, T, S, H_q, H_kv, d,
                    k, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws) if nb else 0,
                    ws.numel() if (nb and ws is not None) else 0, _stream())
    return (out, lse) if with_lse else out


def indexshare_group(q_I, k_I, w, q_pos0, kv_len, k, layers, sm_scale, with_lse=False,
                     ws=None, idx=None, outs=None):
    """One selection for the group, attention for every layer.

    layers: list of dicts with q, K, V device tensors.  Returns (idx, [out per layer])
    (and [lse per layer] when with_lse).
    """
    torch = _torch()
    a = indexer_args(q_I, k_I, w, q_pos0, kv_len)
    q0 = layers[0]["q"]
    B, T, H_q, d = q0.shape
    H_kv = layers[0]["K"].shape[2]
    if idx is None:
        idx = torch.empty((a.B, a.T, k), dtype=torch.int32, device=q_I.device)
    if outs is None:
        outs = [torch.empty_like(L["q"]) for L in layers]
    lses = ([torch.empty((B, T, H_q), dtype=torch.float32, device=q0.device) for _ in layers]
            if with_lse else None)
    nb = indexshare_workspace_bytes(a, k, H_q, H_kv, d)
    if ws is None or ws.numel() < nb:
        ws = workspace(nb, q_I.device)
    indexshare_group_fwd(a, k, len(layers), [_ptr(L["q"]) for L in layers],
                         [_ptr(L["K"]) for L in layers], [_ptr(L["V"]) for L in layers],
                         [_ptr(o) for o in outs], [_ptr(x) for x in lses] if lses else None,
                         H_q, H_kv, d, float(sm_scale), _ptr(idx), _ptr(ws), ws.numel(),
                         _stream())
    return (idx, outs, lses) if with_lse else (idx, outs)


def group_attention(layers, idx, sm_scale, kv_len=None, with_lse=False, ws=None):
    """The attention of every layer over one selection (sparse_attn_group_fwd): layers is a
    list of dicts with q, K, V device tensors; returns [out] (and [lse]) per layer."""
    torch = _torch()
    q0 = layers[0]["q"]
    B, T, H_q, d = q0.shape
    S, H_kv = layers[0]["K"].shape[1], layers[0]["K"].shape[2]
    k = idx.shape[2]
    for L in layers:
        for t in (L["q"], L["K"], L["V"]):
            assert t.is_contiguous(), "attention tensors must be contiguous"
    outs = [torch.empty_like(L["q"]) for L in layers]
    lses = ([torch.empty((B, T, H_q), dtype=torch.float32, device=q0.device) for _ in layers]
            if with_lse else None)
    nb = sparse_attn_group_workspace_bytes(B, T, H_q, H_kv, d, k, len(layers))
    if ws is None and nb:
        ws = workspace(nb, q0.device)
    sparse_attn_group_fwd(len(layers), [_ptr(L["q"]) for L in layers], [_ptr(L["K"]) for L in layers],
                          [_ptr(L["V"]) for L in layers], [_ptr(o) for o in outs],
                          [_ptr(x) for x in lses] if lses else None, _ptr(idx), _ptr(kv_len), B,
                          T, S, H_q, H_kv, d, k, float(sm_scale), _ptr(ws) if ws is not None else 0,
                          nb, _stream())
    return (outs, lses) if with_lse else outs


def append_kv(pos0, k_I_new=None, k_I_cache=None, K_new=None, V_new=None, K_cache=None,
              V_cache=None):
    """Writes new tokens into the caches in place at positions pos0[b] + t: indexer keys
    (fp32 [B,T_new,d_I]) rounded to e4m3 into k_I_cache (u8 [B,S,d_I]); K/V rows (bf16
    [B,T_new,H_kv,d]) into K_cache/V_cache (bf16 [B,S,H_kv,d])."""
    ref_new = k_I_new if k_I_new is not None else (K_new if K_new is not None else V_new)
    ref_cache = k_I_cache if k_I_cache is not None else (K_cache if K_cache is not None else V_cache)
    B, T_new = ref_new.shape[0], ref_new.shape[1]
    S = ref_cache.shape[1]
    d_I = k_I_new.shape[2] if k_I_new is not None else 0
    kv = K_new if K_new is not None else V_new
    H_kv, d = (kv.shape[2], kv.shape[3]) if kv is not None else (0, 0)
    for t in (k_I_new, K_new, V_new, k_I_cache, K_cache, V_cache, pos0):
        assert t is None or t.is_contiguous(), "append tensors must be contiguous"
    ix_append_kv(_ptr(k_I_new), _ptr(K_new), _ptr(V_new), _ptr(pos0), B, T_new, S, d_I, H_kv, d,
                 _ptr(k_I_cache), _ptr(K_cache), _ptr(V_cache), _stream())


def pool_keys(k_I, kv_len, pool=4):
    """Block keys u8 [B, ceil(S/pool), d_I] from FP8 indexer keys u8 [B, S, d_I]."""
    torch = _torch()
    B, S, D = k_I.shape
    out = torch.empty((B, (S + pool - 1) // pool, D), dtype=torch.uint8, device=k_I.device)
    ix_pool_keys(_ptr(k_I), _ptr(kv_len), B, S, D, pool, _ptr(out), _stream())
    return out


def topk_pooled(q_I, k_pooled, w, q_pos0, kv_len, S_max, pool, k_blocks, ws=None):
    """idx int32 [B, T, k_blocks * pool]: token positions of the best k_blocks blocks."""
    torch = _torch()
    B, T, H, D = q_I.shape
    for t in (q_I, k_pooled, w, q_pos0, kv_len):
        assert t.is_contiguous(), "indexer tensors must be contiguous"
    a = IndexerArgs(_ptr(q_I), _ptr(k_pooled), _ptr(w), _ptr(q_pos0), _ptr(kv_len), B, T, S_max,
                    H, D)
    idx = torch.empty((B, T, k_blocks * pool), dtype=torch.int32, device=q_I.device)
    nb = ix_topk_pooled_workspace_bytes(a, pool, k_blocks)
    if ws is None or ws.numel() < nb:
        ws = workspace(nb, q_I.device)
    ix_topk_pooled(a, pool, k_blocks, _ptr(idx), _ptr(ws), ws.numel(), _stream())
    return idx


def sparse_attention_backward(q, K, V, idx, out, lse, dout, sm_scale, kv_len=None,
                              rows_per_pass=None, pair_rows=PAIR_ROWS_BF16):
    """(dq fp32 [B,T,H_q,d], dK fp32 [B,S,H_kv,d], dV fp32 [B,S,H_kv,d]) of
    sparse_attention(q, K, V, idx) for the given dout (out, lse: its forward outputs).
    rows_per_pass: None adds dK / dV with atomics; a row count takes the atomic-free form
    with a workspace for passes of that many query rows, its pair rows in the precision
    pair_rows names (PAIR_ROWS_BF16 or PAIR_ROWS_FP32)."""
    torch = _torch()
    B, T, H_q, d = q.shape
    S, H_kv = K.shape[1], K.shape[2]
    k = idx.shape[2]
    for t in (q, K, V, idx, out, lse, dout):
        assert t.is_contiguous(), "attention tensors must be contiguous"
    dq = torch.empty((B, T, H_q, d), dtype=torch.float32, device=q.device)
    dK = torch.zeros((B, S, H_kv, d), dtype=torch.float32, device=q.device)
    dV = torch.zeros((B, S, H_kv, d), dtype=torch.float32, device=q.device)
    ws, nb = None, 0
    if rows_per_pass is not None:
        nb = sparse_attn_bwd_workspace_bytes(B, T, S, H_kv, d, k, rows_per_pass, pair_rows)
        ws = workspace(nb, q.device)
    sparse_attn_bwd(_ptr(q), _ptr(K), _ptr(V), _ptr(idx), _ptr(kv_len), _ptr(out), _ptr(lse),
                    _ptr(dout), B, T, S, H_q, H_kv, d, k, float(sm_scale), _ptr(dq), _ptr(dK),
                    _ptr(dV), pair_rows, _ptr(ws) if ws is not None else 0, nb, _stream())
    return dq, dK, dV


def group_attention_backward(idx, layers, sm_scale, kv_len=None, rows_per_pass=None,
                             pair_rows=PAIR_ROWS_BF16):
    """The attention backward of every layer of an IndexShare group over the shared idx,
    atomic-free with the selection inverted once per pass.  layers: list of dicts with q, K,
    V, out, lse, dout device tensors.  Returns [(dq, dK, dV) per layer].  rows_per_pass:
    None takes all rows in one pass; pair_rows: the precision of the pair rows."""
    torch = _torch()
    q0 = layers[0]["q"]
    B, T, H_q, d = q0.shape
    S, H_kv = layers[0]["K"].shape[1], layers[0]["K"].shape[2]
    k = idx.shape[2]
    grads = [(torch.empty((B, T, H_q, d), dtype=torch.float32, device=q0.device),
              torch.zeros((B, S, H_kv, d), dtype=torch.float32, device=q0.device),
              torch.zeros((B, S, H_kv, d), dtype=torch.float32, device=q0.device)) for _ in layers]
    nb = sparse_attn_bwd_workspace_bytes(B, T, S, H_kv, d, k, rows_per_pass or B * T, pair_rows)
    ws = workspace(nb, q0.device)
    names = ("q", "K", "V", "out", "lse", "dout")
    ptrs = [[_ptr(L[n]) for L in layers] for n in names]
    indexshare_group_bwd(_ptr(idx), _ptr(kv_len), len(layers), *ptrs, B, T, S, H_q, H_kv, d, k,
                         float(sm_scale), [_ptr(g[0]) for g in grads], [_ptr(g[1]) for g in grads],
                         [_ptr(g[2]) for g in grads], pair_rows, _ptr(ws), nb, _stream())
    return grads


def ix_indexer_bwd(args: IndexerArgs, k: int, idx: int, dscores: int, dq_I: int, dw: int,
                   dk_I: int, pair_rows: int = 0, ws: int = 0, ws_bytes: int = 0,
                   stream: int = 0):
    _check(load().ix_indexer_bwd(ctypes.byref(args), k, idx, dscores, dq_I, dw, dk_I, pair_rows,
                                 ws, ws_bytes, stream))


def ix_indexer_bwd_workspace_bytes(args: IndexerArgs, k: int, rows_per_pass: int,
                                   pair_rows: int = 0) -> int:
    return load().ix_indexer_bwd_workspace_bytes(ctypes.byref(args), k, rows_per_pass, pair_rows)


def indexer_bwd(args: IndexerArgs, idx, dscores, device, rows_per_pass=None,
                pair_rows=PAIR_ROWS_BF16):
    """(dq_I fp32 [B,T,H_I,d_I], dw fp32 [B,T,H_I], dk_I fp32 [B,S_max,d_I]): the indexer
    inputs' gradients from d loss / d sel_scores (dk_I starts from zero here).
    rows_per_pass: None adds dk_I with atomics; a row count takes the atomic-free form
    with a workspace for passes of that many query rows, its dk_I rows in the precision
    pair_rows names."""
    torch = _torch()
    for t in (idx, dscores):
        assert t.is_contiguous(), "indexer backward tensors must be contiguous"
    assert dscores.dtype == torch.float32 and tuple(dscores.shape) == tuple(idx.shape)
    B, T, H, D, S = args.B, args.T, args.H_I, args.d_I, args.S_max
    dq = torch.empty((B, T, H, D), dtype=torch.float32, device=device)
    dw = torch.empty((B, T, H), dtype=torch.float32, device=device)
    dk = torch.zeros((B, S, D), dtype=torch.float32, device=device)
    ws, nb = None, 0
    if rows_per_pass is not None:
        nb = ix_indexer_bwd_workspace_bytes(args, idx.shape[2], rows_per_pass, pair_rows)
        ws = workspace(nb, device)
    ix_indexer_bwd(args, idx.shape[2], _ptr(idx), _ptr(dscores), _ptr(dq), _ptr(dw), _ptr(dk),
                   pair_rows, _ptr(ws), nb, _stream())
    return dq, dw, dk


def indexer_kl(q, K, idx, lse, sel_scores, sm_scale, kv_len=None):
    """(loss fp32 [B,T], dscores fp32 [B,T,k]) of the indexer's KL objective: the target is
    the head-summed attention probabilities exp(sm_scale q.K_j - lse) over the selection,
    normalised; the prediction is the softmax of sel_scores."""
    torch = _torch()
    B, T, H_q, d = q.shape
    S, H_kv = K.shape[1], K.shape[2]
    k = idx.shape[2]
    for t in (q, K, idx, lse, sel_scores):
        assert t.is_contiguous(), "KL tensors must be contiguous"
    assert lse.dtype == torch.float32 and sel_scores.dtype == torch.float32
    loss = torch.empty((B, T), dtype=torch.float32, device=q.device)
    dsc = torch.empty((B, T, k), dtype=torch.float32, device=q.device)
    ix_indexer_kl(_ptr(q), _ptr(K), _ptr(idx), _ptr(kv_len), _ptr(lse), _ptr(sel_scores), B, T, S,
                  H_q, H_kv, d, k, float(sm_scale), _ptr(loss), _ptr(dsc), _stream())
    return loss, dsc
