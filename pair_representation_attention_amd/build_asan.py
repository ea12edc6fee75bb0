"""Host-sanitized build of libpairattn.so for checking the host-side code.

The C ABI's validation, workspace sizing and argument marshalling run on the
host.  This builds a copy of the library whose host code (pairattn_api.hip,
where that logic lives) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer; device code is built as usual (each sanitizer flag
is scoped to the host pass with -Xarch_host).  The other objects come from the
regular build.  Load it with the sanitizer runtime preloaded:

    LD_PRELOAD=$(python -m pair_representation_attention_amd.build_asan --runtime) \\
    PAIRATTN_LIB=$(python -m pair_representation_attention_amd.build_asan) \\
    ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_abi_host.py
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as _b

OUT = os.path.join(_b.PKG, "_build", "asan", "libpairattn_asan.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def runtime() -> str:
    """The shared ASan runtime of the ROCm clang (it carries the UBSan handlers)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_b.hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(cand):
            path = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                                  text=True, check=True).stdout.strip()
            if os.path.exists(path):
                return path
    raise RuntimeError("libclang_rt.asan-x86_64.so not found")


def build(verbose: bool = False) -> str:
    cc = _b.hipcc()
    objdir = os.path.join(_b.PKG, "_build")
    others = [os.path.join(objdir, s.replace(".hip", ".o")) for s in _b.SOURCES if s != "pairattn_api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        _b.build(verbose=verbose)
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    api = os.path.join(os.path.dirname(OUT), "pairattn_api_asan.o")
    cmd = [cc, *_b.compile_flags(), *HOST_SAN, "-c", os.path.join(_b.CSRC, "pairattn_api.hip"), "-o", api]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    cmd = [cc, f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", "-shared-libasan", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", api, *others, "-o", OUT]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    return OUT


if __name__ == "__main__":
    print(runtime() if "--runtime" in sys.argv else build(verbose="-v" in sys.argv))
