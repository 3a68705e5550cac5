"""Compile the HIP library (libdflash.so, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdflash.so")
# source, extra flags: the int4 kernels and the attention keep MFMA results in
# VGPRs (their results are rescaled in VALU at once)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCES = [("kernels.hip", []), ("skinny.hip", VGPR_FORM), ("stream.hip", VGPR_FORM),
           ("attention.hip", VGPR_FORM), ("settle.hip", VGPR_FORM), ("batch.hip", VGPR_FORM),
           ("route.hip", []),
           ("dflash.cpp", [])]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 VALU ops in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
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


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory() as tmpdir:
        objs = []
        for src, extra in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            _run(["hipcc", *FLAGS, *extra, *inc, "-c", "-x", "hip", os.path.join(CSRC, src),
                  "-o", obj], verbose)
            objs.append(obj)
        tmp = LIB + ".tmp"
        _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
