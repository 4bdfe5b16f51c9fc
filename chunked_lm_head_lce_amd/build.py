"""Build the gfx950 shared library (liblce.so) in-tree with hipcc.

Usage: python -m chunked_lm_head_lce_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblce.so")
SOURCES = ["lce_kernels.hip", "lce_api.cpp", "lce_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (need ROCm with gfx950 support)")


def compile_command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 instructions are kept out of all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # one lane's tile-claiming atomic must not become a wave-wide
        # reduction that waits for its result where it is issued
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-I", os.path.join(ROOT, "include"),
        *(extra or []),
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
