"""Builds libsas.so (the C ABI in include/sas.h) for gfx950 with hipcc, in-tree.

    python -m learned_context_ranking_amd.build_lib      # or __graft_entry__.build()

Objects go to ``_build/`` at the repository root; the shared library is written next to
this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsas.so")
SOURCES = ["sas_api.hip", "select.hip", "attn_fwd.hip", "attn_bwd.hip", "decode.hip", "decode_select.hip",
           "profile.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -packed-fp32-ops keeps the compiler from forming packed fp32 VALU instructions.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libsas_asan.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime shipped with ROCm's LLVM (for LD_PRELOAD)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


def build_asan(verbose: bool = False) -> str:
    """The same library with AddressSanitizer on its host code only (the device code is
    built as usual): checks the C ABI layer's argument checks, error strings, workspace
    queries and measurement bookkeeping for host memory errors. Written to _build/asan/."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                "-Xarch_host", "-fsanitize=address"]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(ASAN_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "-shared-libasan", *objs, "-o", ASAN_LIB], verbose)
    return ASAN_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
