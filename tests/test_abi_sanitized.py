"""The host-side ABI tests again, against a build whose host code (abi.cpp: argument validation,
size arithmetic, error strings) runs under AddressSanitizer and UndefinedBehaviorSanitizer.

CPU only: the sanitized build is a check of host code, and the tests it runs pass fake device
addresses that must never reach a kernel. Any sanitizer report fails the run (UBSan halts on the
first error, ASan aborts on a bad access).
"""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="the sanitized host build is checked where no GPU is visible")


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_abi_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("g++ sanitizer runtimes not installed")
    from gated_softmax_attention_fox_amd import build
    lib = build.build_sanitized()
    syms = subprocess.run(["nm", "-D", lib], stdout=subprocess.PIPE, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "build is not instrumented"
    env = dict(os.environ, FOX_LIBRARY=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, tail
    assert " passed" in r.stdout, tail
