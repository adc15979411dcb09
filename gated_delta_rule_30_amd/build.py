"""Build libkda.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_chunk.hip", "kda_scan.hip", "kda_bwd.hip", "kda_wide.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into gated_delta_rule_30_amd/libkda.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
