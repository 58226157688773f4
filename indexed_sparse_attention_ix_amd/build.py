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


CHECK_DIR = os.path.join(BUILD, "check")
CHECK_LIB = os.path.join(CHECK_DIR, "libix_check.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only (the device code is
# built as usual, at -O1: this library is never launched from) and the test hook that makes
# launches report a chosen HIP error.  Loaded by the CPU tests of the C ABI.
CHECK_FLAGS = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Wall", "-Wno-unused-command-line-argument", "-fno-omit-frame-pointer",
               "-DIX_TEST_HOOKS", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
               "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of hipcc's clang (preloaded into a Python that
    loads the check library)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"AddressSanitizer runtime not found ({path!r})")
    return path


def build_check() -> str:
    """Builds _build/check/libix_check.so (sanitized host code, test hooks) from csrc/;
    sources unchanged since the last build are not compiled again."""
    os.makedirs(CHECK_DIR, exist_ok=True)

    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    headers += [os.path.join(os.path.dirname(PKG), "include", "ix.h")]
    newest_header = max(os.path.getmtime(h) for h in headers)
    stamp = os.path.join(CHECK_DIR, "flags")
    flags = " ".join(CHECK_FLAGS)
    if not os.path.exists(stamp) or open(stamp).read() != flags:
        newest_header = float("inf")  # other flags: compile everything again

    def one(src):
        obj = os.path.join(CHECK_DIR, os.path.basename(src) + ".o")
        if os.path.exists(obj) and os.path.getmtime(obj) > max(os.path.getmtime(src), newest_header):
            return obj
        r = subprocess.run([HIPCC, *CHECK_FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (check build) failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj
    srcs = sources(CSRC)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    tmp = CHECK_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"check link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CHECK_LIB)
    with open(stamp, "w") as f:
        f.write(flags)
    return CHECK_LIB


if __name__ == "__main__":
    build()
