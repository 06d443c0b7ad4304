"""Build libmoe.so (HIP for gfx950) in-tree: one hipcc compile per source, then a shared link.

Usage: python -m mixture_experts_layer_14_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["api.hip", "router.hip", "dispatch.hip", "experts.hip", "gemm_stream.hip", "gemm_wide.hip", "gemm_ring.hip",
           "gemm_wstream.hip", "gemm_wstream_fp8.hip",
           "gemm_wide_fp8.hip", "combine.hip", "decode_fused.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep packed fp32 instructions out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so; returns its path. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-o", tmp, *objs])
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
