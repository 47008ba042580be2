"""Build the HIP library ``libep.so`` for gfx950 with hipcc, in-tree, and
the benchmark's bandwidth-ceiling kernels ``libep_ceilings.so`` beside it.

    python -m combine_ep_layout_08_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libep.so")
CEILINGS_LIB = os.path.join(PKG, "libep_ceilings.so")
CEILINGS_SOURCES = ["ep_ceilings.hip"]

SOURCES = ["ep_api.cpp", "ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_backward.hip",
           "ep_rank.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, extra=(), verbose: bool = False, sources=None) -> str:
    """Compile every HIP source and the C ABI into one shared library."""
    srcs = [os.path.join(CSRC, s) for s in (sources or SOURCES)]
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           "-o", tmp, "-x", "hip", *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)
    return out


def build_ceilings(out: str = CEILINGS_LIB, verbose: bool = False) -> str:
    """Compile the bandwidth-ceiling kernels (benchmark only)."""
    return build(out, verbose=verbose, sources=CEILINGS_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceilings(verbose=True))
