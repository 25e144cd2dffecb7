"""Build the HIP library ``libmla.so`` in-tree for gfx950 (MI355X).

Every call recompiles.  The library is a plain shared object with a C ABI
(``include/mla.h``); no torch headers are involved.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla.so")
SOURCES = ["api.cpp", "attn_mfma.hip", "attn_generic.hip", "proj.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MLA library)")


def compile_cmd(out: str = LIB) -> list:
    return [
        hipcc(), "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
        # no packed fp32 instructions anywhere
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # score MFMAs accumulate in VGPRs; the O accumulator is pinned to AGPRs by asm
        "-mllvm", "-amdgpu-mfma-vgpr-form=true",
        "-I", os.path.join(ROOT, "include"),
        "-x", "hip", *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = compile_cmd(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose and (res.stdout or res.stderr):
        print(res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
