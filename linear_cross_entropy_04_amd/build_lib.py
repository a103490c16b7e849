"""Build libflce.so (gfx950) in-tree with hipcc.

Run ``python -m linear_cross_entropy_04_amd.build_lib`` or call ``build()``.
Objects go to ``_build/`` at the repository root; the library lands next to
this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libflce.so")
SOURCES = ["flce_api.hip", "gemm_bf16.hip", "kernels_f32.hip", "kernels_common.hip",
           "ce_kernels.hip", "pair_kernels.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are disabled for the device code (the host pass
# warns that it does not know the feature; that is expected).
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source and link libflce.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = CFLAGS + list(extra_flags or [])

    def one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
