"""Build libpairattn.so (HIP, gfx950) in-tree with hipcc, and beside it
libpairattn_debug.so: the same sources at -O1 with -DPA_DEBUG, whose kernels
check the indices they compute (pairattn_debug_status reads the result).

Usage:  python -m pair_representation_attention_amd.build [--release-only]
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
DEBUG_LIB = os.path.join(PKG, "libpairattn_debug.so")

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
        *(["-O1", "-DPA_DEBUG"] if debug else ["-O3"]),
        "-std=c++17",
        "-fPIC",
        # packed fp32 VALU forms are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-munsafe-fp-atomics",
        "-Wno-unused-result",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def _build_one(debug: bool, verbose: bool) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build", "debug" if debug else "")
    os.makedirs(objdir, exist_ok=True)
    out = DEBUG_LIB if debug else LIB
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *compile_flags(debug), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print("[build]", " ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = True, with_debug: bool = True) -> str:
    """Both libraries (the debug one unless with_debug is False); returns the
    release library's path."""
    lib = _build_one(False, verbose)
    if with_debug:
        _build_one(True, verbose)
    return lib


if __name__ == "__main__":
    build(with_debug="--release-only" not in sys.argv)
