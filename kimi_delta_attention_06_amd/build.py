"""Build the KDA HIP library (libkda.so) in-tree for gfx950 with hipcc.

Every source compiles to an object in parallel, then one link step produces
kimi_delta_attention_06_amd/libkda.so.  Usage: python -m kimi_delta_attention_06_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
BUILD_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops are disabled for all device code (see the design notes on
# gfx950 packed fp32); -O3, C++17, no fast-math (IEEE division and exp).
FLAGS = ["-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]
# (source, object name, flags of its own).  kda_chunk.hip is built twice: its fused-forward
# part with the matrix-core-ILP instruction scheduler (2.5% faster on the Kimi-Linear
# layer, 6% on a 1M-token sequence, bit-identical results), and its split-path part with
# the default scheduler (the ILP one slows the split path's passes by ~6%).  The fused
# part is also built for XNACK off only (gfx950:xnack-): the compiler then need not keep
# the address registers of a memory clause live for a replay, which takes another 1.4%
# off the Kimi-Linear layer; the split and decode kernels gain nothing from it (the split
# passes lose ~2%), so they keep the XNACK-agnostic target.  A process that turns XNACK on
# cannot load the fused kernels: their entry points then return KDA_ERR_LAUNCH.  The
# chunkwise backward's two kernels are built with LLVM's iterative ILP scheduler (1.8% off
# the Kimi-Linear layer's backward, bit-identical gradients; max-ilp gains 0.3%).
SOURCES = [
    ("kda_api.cpp", "kda_api.o", []),
    ("kda_recurrent.hip", "kda_recurrent.o", []),
    ("kda_chunk.hip", "kda_chunk_fused.o", ["--offload-arch=" + ARCH + ":xnack-", "-DKDA_CHUNK_SPLIT=0",
                                            "-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
    ("kda_chunk.hip", "kda_chunk_split.o", ["-DKDA_CHUNK_FUSED=0"]),
    ("kda_backward.hip", "kda_backward.o", []),
    ("kda_backward_chunk.hip", "kda_backward_chunk.o", ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]),
]


def _compile(entry, extra) -> str:
    src, name, own = entry
    obj = os.path.join(BUILD_DIR, name)
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    arch = [] if any(f.startswith("--offload-arch=") for f in own) else ["--offload-arch=" + ARCH]
    cmd = [HIPCC] + FLAGS + arch + list(own) + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out:
        print(out, file=sys.stderr)
    return obj


def build(extra_flags=(), verbose: bool = True) -> str:
    """Compile every HIP source and link libkda.so; always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
