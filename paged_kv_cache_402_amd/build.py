"""Builds libpagedkv.so in-tree with hipcc for gfx950.

    python paged_kv_cache_402_amd/build.py [-v]      (or __graft_entry__.build())

Each source compiles to an object under _build/ (in parallel), then one link produces
paged_kv_cache_402_amd/libpagedkv.so, written under a temporary name and renamed into place.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpagedkv.so")

SOURCES = ["decode.hip", "decode_step.hip", "decode_groups.hip", "prefix.hip", "cache_ops.hip",
           "probe.hip", "static_ws.hip", "capi.cpp", "shapes.cpp", "block_manager.cpp",
           "scheduler.cpp", "pool_plan.cpp", "errors.cpp"]
ARCH = "gfx950"

COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# Device code: keep hipcc from forming packed fp32 instructions (v_pk_*_f32).
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked in $HIPCC, /opt/rocm/bin, PATH)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS
    if src.endswith(".hip"):
        cmd += DEVICE_FLAGS
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (src, r.stdout, r.stderr))
    if verbose and r.stderr:
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source and links libpagedkv.so; returns its path. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
