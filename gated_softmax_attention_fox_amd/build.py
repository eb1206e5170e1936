"""Build libfox.so (gfx950) in-tree with hipcc.

    python -m gated_softmax_attention_fox_amd.build

Compiles every csrc/*.hip and csrc/*.cpp into _build/ and links
gated_softmax_attention_fox_amd/libfox.so. Always recompiles.
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
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
