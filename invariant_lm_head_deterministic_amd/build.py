"""Build the gfx950 HIP library ``librlk_logprob.so`` in-tree with hipcc.

The numeric contract depends on these flags: -ffp-contract=off (no fused multiply-add is formed
from separate operations), -fno-fast-math, denormals kept, fp32 division and square root correctly rounded, and no
packed-fp32 instructions.
"""

from __future__ import annotations

import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librlk_logprob.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["rlk_kernels.hip", "rlk_backward.hip", "rlk_host.hip"]

CONTRACT_FLAGS = [
    "-O3",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def flags() -> list[str]:
    return ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"] + CONTRACT_FLAGS


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library; returns its path."""
    objs = []
    fp = " ".join(CONTRACT_FLAGS)
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [HIPCC, *flags(), f'-DRLK_BUILD_FLAGS="{fp}"', "-c", os.path.join(CSRC, src),
               "-o", obj]
        if verbose:
            print(" ".join(shlex.quote(c) for c in cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
