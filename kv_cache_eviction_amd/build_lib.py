"""Builds ``libh2o.so`` (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed-fp32 code generation
turned off (the kernels are written with scalar fp32 arithmetic).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libh2o.so")
SOURCES = ["attn_fwd.hip", "decode.hip", "score.hip", "select_scatter.hip", "attn_bwd.hip", "recurrence.hip", "api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(verbose: bool = True) -> str:
    """Compiles every source (in parallel) and links ``kv_cache_eviction_amd/libh2o.so``."""
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = False
    for cmd, p in procs:
        out, _ = p.communicate()
        # the host pass does not know the gfx950-only feature flag; that note is harmless
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if verbose and lines:
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            print("FAILED: " + " ".join(cmd), file=sys.stderr)
            failed = True
    if failed:
        raise RuntimeError("hipcc compilation failed")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        print(r.stdout, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
