"""Builds libkda.so (HIP, gfx950) in-tree with hipcc.

    python -m gated_delta_rule_chunkwise_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_chunk.hip", "kda_chunk2.hip", "kda_fused.hip", "kda_decode.hip", "kda_bwd.hip",
           "kda_noalloc.hip"]

# The packed fp32 VALU forms are switched off for the device code, which is
# written with scalar or float2 arithmetic only; hipcc's host pass warns that it
# does not know the feature.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile_cmd(src: str, obj: str) -> list:
    if src.endswith(".cpp"):
        return [hipcc(), "-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"),
                "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    return [hipcc()] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                   "-c", os.path.join(CSRC, src), "-o", obj]


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(len(SOURCES), n, 16))


def build(verbose: bool = False) -> str:
    """Compiles every source (in parallel, one hipcc per file) and links libkda.so."""
    tag = ".%d" % os.getpid()
    objs = [os.path.join(CSRC, os.path.splitext(src)[0] + tag + ".o") for src in SOURCES]
    cmds = [_compile_cmd(src, obj) for src, obj in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)

    def run(cmd):
        return subprocess.run(cmd, stderr=None if verbose else subprocess.PIPE, text=True)

    try:
        with ThreadPoolExecutor(_jobs()) as ex:
            results = list(ex.map(run, cmds))
        for cmd, r in zip(cmds, results):
            if r.returncode != 0:
                raise subprocess.CalledProcessError(r.returncode, cmd, stderr=r.stderr)
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, check=True)
        os.replace(tmp, LIB)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
