"""Build libkda.so in-tree with hipcc for gfx950.

Each source compiles to its own object in parallel (gated_delta_rule_30_amd/_build/), then one
hipcc call links the shared library. Every call recompiles everything.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_chunk.hip", "kda_scan.hip", "kda_bwd.hip",
           "kda_wide.hip", "kda_noalloc.hip", "kda_prologue.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result",
]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    return r.returncode, err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source into gated_delta_rule_30_amd/libkda.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    tag = "%d" % os.getpid()
    cmds, objs = [], []
    for s in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".%s.o" % tag)
        objs.append(obj)
        cmds.append([HIPCC] + FLAGS + inc + ["-c", os.path.join(CSRC, s), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, err) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError("hipcc failed (%d):\n%s" % (rc, err))
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp%s" % tag
    rc, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    for o in objs:
        os.remove(o)
    if rc != 0:
        raise RuntimeError("hipcc link failed (%d):\n%s" % (rc, err))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
