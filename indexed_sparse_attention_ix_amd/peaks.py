"""ctypes binding of libix_peaks.so (include/ix_peaks.h): the measured-ceiling microbenchmarks
the benchmark reads kernel times against.  Not part of the path; raises if the library is not
built."""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p

from .binding import IxError

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libix_peaks.so")

# every symbol include/ix_peaks.h declares
EXPORTS = ("ix_peak_last_error", "ix_peak_mfma_fp8", "ix_peak_copy", "ix_peak_read",
           "ix_peak_gather", "ix_peak_gather_wide", "ix_peak_gather_selection", "ix_peak_atomic_add")

_lib = None


def load(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libix_peaks.so not built at {path}; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    L.ix_peak_last_error.restype = ctypes.c_char_p
    L.ix_peak_last_error.argtypes = []
    L.ix_peak_mfma_fp8.restype = c_int32
    L.ix_peak_mfma_fp8.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]
    L.ix_peak_copy.restype = c_int32
    L.ix_peak_copy.argtypes = [c_void_p, c_void_p, c_size_t, c_void_p]
    L.ix_peak_read.restype = c_int32
    L.ix_peak_read.argtypes = [c_void_p, c_size_t, c_int32, c_int32, c_void_p, c_void_p]
    L.ix_peak_gather.restype = c_int32
    L.ix_peak_gather.argtypes = [c_void_p, c_size_t, c_void_p, c_int64, c_int32, c_void_p, c_void_p]
    L.ix_peak_gather_wide.restype = c_int32
    L.ix_peak_gather_wide.argtypes = [c_void_p, c_size_t, c_int32, c_void_p, c_int64, c_int32,
                                      c_int32, c_void_p, c_void_p]
    L.ix_peak_gather_selection.restype = c_int32
    L.ix_peak_gather_selection.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p] + [c_int32] * 8 + \
        [c_void_p, c_void_p]
    L.ix_peak_atomic_add.restype = c_int32
    L.ix_peak_atomic_add.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_void_p]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise IxError(status, load().ix_peak_last_error().decode(errors="replace"))


def ix_peak_mfma_fp8(operands, valu_per_mfma, blocks, iters, out, stream=0):
    _check(load().ix_peak_mfma_fp8(operands, valu_per_mfma, blocks, iters, out, stream))


def ix_peak_copy(src, dst, nbytes, stream=0):
    _check(load().ix_peak_copy(src, dst, nbytes, stream))


def ix_peak_read(src, nbytes, blocks, nontemporal, out, stream=0):
    _check(load().ix_peak_read(src, nbytes, blocks, nontemporal, out, stream))


def ix_peak_gather(table, table_bytes, rows, n, blocks, out, stream=0):
    _check(load().ix_peak_gather(table, table_bytes, rows, n, blocks, out, stream))


def ix_peak_gather_wide(table, seg_bytes, n_seg, rows, n, blocks, nontemporal, out, stream=0):
    _check(load().ix_peak_gather_wide(table, seg_bytes, n_seg, rows, n, blocks, nontemporal, out,
                                      stream))


def ix_peak_gather_selection(kc, vc, idx, kv_len, B, T, S_max, H_kv, d, k, splits, blocks_per_cu,
                             out, stream=0):
    _check(load().ix_peak_gather_selection(kc, vc, idx, kv_len, B, T, S_max, H_kv, d, k, splits,
                                           blocks_per_cu, out, stream))


def ix_peak_atomic_add(table, rows, idx, n, stream=0):
    _check(load().ix_peak_atomic_add(table, rows, idx, n, stream))
