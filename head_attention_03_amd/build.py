"""Compile libfmha.so for gfx950 with hipcc, in place (next to this file).

    python -m head_attention_03_amd.build

Every call recompiles.  The flags keep hipcc from forming packed-fp32 instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "fmha_fwd.hip"), os.path.join(HERE, "csrc", "fmha_splitkv.hip"),
           os.path.join(HERE, "csrc", "fmha_bwd.hip")]
LIB = os.path.join(HERE, "libfmha.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
