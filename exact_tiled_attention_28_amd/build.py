"""Build libfa.so (the C-ABI attention library) for gfx950 with hipcc.

Usage: python -m exact_tiled_attention_28_amd.build [--verbose]

The library is built in-tree at exact_tiled_attention_28_amd/lib/libfa.so.
Every HIP source is compiled with packed-fp32 instruction generation turned
off (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libfa.so")
ROOT = os.path.dirname(PKG)

HIP_SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip"]
HOST_SOURCES = ["fa_api.cpp"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    if verbose and (res.stdout or res.stderr):
        sys.stderr.write(res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source and link libfa.so; returns its path."""
    cc = hipcc()
    os.makedirs(LIBDIR, exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        objs = []
        for src in HIP_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([cc, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([cc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libfa.so")
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        shutil.move(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
