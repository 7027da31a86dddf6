"""Build the SSA HIP library (libssa.so) for gfx950 with hipcc.

Usage: python -m block_sparse_full_amd.build   (or call build_library()).
       python -m block_sparse_full_amd.build --host-asan   (C-ABI host code
       under AddressSanitizer, for the host sanitizer test)
Objects go to _build/ at the repository root; the shared library lands next
to this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssa.so")
SOURCES = ["ssa_select.hip", "ssa_attn_prefill.hip", "ssa_attn_decode.hip", "ssa_loss.hip",
           "ssa_attn_backward.hip", "ssa_api.hip"]
# The attention kernels never see NaNs (finite inputs; masked logits are
# -inf), so let max() skip NaN canonicalisation.
FILE_FLAGS = {"ssa_attn_prefill.hip": ["-fno-honor-nans"], "ssa_attn_backward.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function",
          # keep the compiler from emitting packed fp32 VALU instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libssa.so)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build_library(verbose: bool = False, extra_flags=()) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        err = _run([cc, *CFLAGS, *FILE_FLAGS.get(src, []), *extra_flags, "-c",
                    os.path.join(CSRC, src), "-o", obj])
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_host_asan_library(verbose: bool = False) -> str:
    """libssa_asan.so under _build/asan: the C-ABI layer (argument checks,
    workspace sizing, layout arithmetic, error strings) compiled with
    AddressSanitizer on its host pass only, linked with the ordinary kernel
    objects. GPU code is never instrumented. Load it in a process that has the
    clang ASan runtime preloaded."""
    cc = hipcc()
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o"))
               for s in SOURCES):
        build_library(verbose=verbose)
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    api = "ssa_api.hip"
    obj = os.path.join(out_dir, "ssa_api.o")
    err = _run([cc, *CFLAGS, "-O1", "-g", "-Xarch_host", "-fsanitize=address",
                "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, api), "-o", obj])
    if verbose and err.strip():
        print(err, file=sys.stderr)
    objs = [obj] + [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != api]
    lib = os.path.join(out_dir, "libssa_asan.so")
    tmp = lib + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


def asan_runtime() -> str | None:
    """Path of the clang ASan runtime that matches hipcc's host compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for c in (clang, shutil.which("clang")):
        if c and os.path.exists(c):
            r = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"],
                               capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return None


if __name__ == "__main__":
    if "--host-asan" in sys.argv:
        print(build_host_asan_library(verbose="-v" in sys.argv))
    else:
        print(build_library(verbose="-v" in sys.argv))
