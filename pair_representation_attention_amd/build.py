"""Build libpairattn.so (HIP, gfx950) in-tree with hipcc.

Usage:  python -m pair_representation_attention_amd.build [--debug]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpairattn.so")

SOURCES = ["pairattn_api.hip", "pa_kernels_bf16.hip", "pa_attn.hip", "pa_kernels_f32.hip", "pa_finish_bf16.hip",
           "pa_calib.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags(debug: bool = False):
    return [
        f"--offload-arch={ARCH}",
        "-O1" if debug else "-O3",
        "-std=c++17",
        "-fPIC",
        # packed fp32 VALU forms are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-munsafe-fp-atomics",
        "-Wno-unused-result",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def build(debug: bool = False, verbose: bool = True) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *compile_flags(debug), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print("[build]", " ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(debug="--debug" in sys.argv)
