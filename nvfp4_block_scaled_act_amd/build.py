"""Build the gfx950 library ``libnvfp4.so`` in-tree with hipcc.

Usage: python -m nvfp4_block_scaled_act_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4.so")
ARCH = os.environ.get("NVFP4_OFFLOAD_ARCH", "gfx950")

SOURCES = ["quantize.hip", "prepare.hip", "w4a16.hip", "w4a4.hip", "moe.hip", "stream.hip", "noalloc.hip", "api.cpp"]
# Packed fp32 VALU ops are kept out of the generated code (-packed-fp32-ops).
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument"]


def source_hash() -> str:
    """sha256 (first 16 hex digits) of every source the library is built
    from: the csrc/ files in name order, then include/nvfp4.h.  The build
    embeds it (nvfp4_build_source_hash) so that a loader can tell a library
    built from other sources."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp", ".cpp", ".h")))
    for f in files:
        h.update(f.encode() + b"\0")
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(HERE, "..", "include", "nvfp4.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def _hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def _compile(src: str, src_hash: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, f'-DNVFP4_SOURCE_HASH="{src_hash}"', "-I", os.path.join(HERE, "..", "include"),
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    src_hash = source_hash()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, src_hash), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
