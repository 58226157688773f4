"""Builds the HIP libraries (gfx950) in-tree with hipcc.

Every .hip source under csrc/ is compiled to an object in _build/ (in parallel) and
linked into indexed_sparse_attention_ix_amd/libix.so, the path's library (include/ix.h).
The measured-ceiling microbenchmarks under csrc_peaks/ become libix_peaks.so
(include/ix_peaks.h), a library of their own.  Packed-FP32 VALU instructions are disabled
for the device code (-packed-fp32-ops): the kernels are written with scalar fp32
arithmetic throughout.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
CSRC_PEAKS = os.path.join(PKG, "csrc_peaks")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libix.so")
PEAKS_LIB = os.path.join(PKG, "libix_peaks.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def sources(folder=CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(os.path.dirname(src)) + "_" +
                       os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if err:
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources(CSRC)
    peak_srcs = sources(CSRC_PEAKS)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(peak_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + peak_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build()
