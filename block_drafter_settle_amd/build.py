"""Compile the HIP library (libdflash.so, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdflash.so")
SOURCES = ["kernels.hip", "dflash.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 VALU ops in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature: drop that warning
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (out.stdout + out.stderr).splitlines() if noise not in l)
    if out.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
