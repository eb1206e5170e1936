"""Build libfox.so (gfx950) in-tree with hipcc.

    python -m gated_softmax_attention_fox_amd.build

Compiles every csrc/*.hip and csrc/*.cpp into _build/ and links
gated_softmax_attention_fox_amd/libfox.so, then the plain-C test driver tests/c_abi/fox_c_smoke
against it. Always recompiles.

    python -m gated_softmax_attention_fox_amd.build --sanitized

builds _build/libfox_san.so, the same library with its host code under ASan and UBSan.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfox.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code (hipcc's host pass warns that
# it does not know the feature; that warning is harmless).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfox)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l
                    and "argument unused during compilation" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    jobs = []
    for f in srcs:
        obj = os.path.join(BUILD, f.rsplit(".", 1)[0] + ".o")
        if f.endswith(".hip"):
            cmd = [hipcc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c",
                   os.path.join(CSRC, f), "-o", obj]
        else:
            cmd = [hipcc, *COMMON, "-c", os.path.join(CSRC, f), "-o", obj]
        jobs.append((cmd, obj))
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for out in ex.map(_run, [c for c, _ in jobs]):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o in jobs], "-o", tmp])
    os.replace(tmp, LIB)
    build_c_smoke(hipcc)
    if verbose:
        print("built", LIB, "and", C_SMOKE)
    return LIB


C_SMOKE_SRC = os.path.join(ROOT, "tests", "c_abi", "fox_c_smoke.c")
C_SMOKE = os.path.join(ROOT, "tests", "c_abi", "fox_c_smoke")


def build_c_smoke(hipcc: str) -> str:
    """The plain-C driver of the attention path (a GPU test runs it): gcc, C11, linked against
    libfox.so (found next to the package through its run path) and the HIP runtime."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          f"-I{rocm}/include", f"-I{INCLUDE}", C_SMOKE_SRC, "-o", C_SMOKE, f"-L{PKG}", "-lfox",
          f"-L{rocm}/lib", "-lamdhip64", "-lm",
          "-Wl,-rpath,$ORIGIN/../../gated_softmax_attention_fox_amd", f"-Wl,-rpath,{rocm}/lib"])
    return C_SMOKE


SAN_LIB = os.path.join(BUILD, "libfox_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer"]


def build_sanitized() -> str:
    """A CPU-side check build: the host code (abi.cpp) compiled by g++ with AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the HIP kernel objects of build() (device code is
    not instrumented). Written to _build/libfox_san.so; load it through FOX_LIBRARY with the
    sanitizer runtimes preloaded (the host tests do)."""
    objs = [os.path.join(BUILD, f.rsplit(".", 1)[0] + ".o")
            for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build()
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    san_obj = os.path.join(BUILD, "abi_san.o")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__",
          f"-I{rocm}/include", f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, "abi.cpp"),
          "-o", san_obj])
    _run(["g++", "-shared", *SAN_FLAGS, san_obj, *objs, f"-L{rocm}/lib", f"-Wl,-rpath,{rocm}/lib",
          "-lamdhip64", "-o", SAN_LIB])
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized())
    else:
        build(verbose="-q" not in sys.argv)
