"""Build libfalcon.so in-tree with hipcc for gfx950.

    python -m weight_recurrent_memory_amd.build_lib      (or __graft_entry__.build())

Every HIP source is compiled with packed-fp32 instruction selection disabled
(the compiler then never emits v_pk_{add,mul,fma}_f32) and linked into one
shared library whose only exported symbols are the C entry points of
include/falcon.h.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libfalcon.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["falcon_api.cpp", "falcon_recurrent.hip", "falcon_decode.hip", "falcon_chunk.hip",
           "falcon_chunk_w1.hip", "falcon_chunk_wy.hip", "falcon_chunk_wyb.hip",
           "falcon_chunk_ip.hip", "falcon_backward.hip", "falcon_masked.hip"]
ARCH = os.environ.get("FALCON_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def flags():
    return ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function"]


def _stale(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")] \
        + [os.path.join(INCLUDE, h) for h in os.listdir(INCLUDE)]
    return max(os.path.getmtime(d) for d in deps) > os.path.getmtime(obj)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and not _stale(src, obj):
        return obj
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (only the stale ones with incremental=True) and link."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda src: _compile(src, incremental), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (res.stdout, res.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
