"""Builds libtria.so (the C-ABI library with the gfx950 kernels) in-tree, and
libtria_probe.so (the streaming-read probe that bench.py --read-probe times).

    python -m key_importance_scoring_amd.build

hipcc cross-compiles for gfx950 without a GPU present.  Packed fp32 VALU ops are
disabled for every HIP translation unit (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtria.so")
PROBE_LIB = os.path.join(HERE, "libtria_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["tria_kernels.hip", "tria_abi.cpp", "tria_stats.cpp"]
PROBE_SOURCES = ["probe_read.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _compile(sources, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile libtria.so and libtria_probe.so (always recompiles); returns libtria.so's path."""
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
