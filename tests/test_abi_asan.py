"""The host-side code of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed): a copy of the library whose host
code is sanitized (pair_representation_attention_amd/build_asan.py) runs the
host ABI tests in a child process with the sanitizer runtime preloaded.  Any
report fails the child (UBSan halts on the first error; ASan always does).
The two tests that import torch are left out: torch is not built for the
preloaded runtime."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_and_ubsan():
    try:
        from pair_representation_attention_amd import build_asan
        rt = build_asan.runtime()
        so = build_asan.build()
    except (RuntimeError, subprocess.CalledProcessError, FileNotFoundError) as e:
        pytest.skip(f"sanitized build unavailable: {e}")
    syms = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, PAIRATTN_LIB=so, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_host.py",
                        "-k", "not no_device and not without_device"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
