"""Build libdv.so (the HIP library behind include/dv.h) in-tree for gfx950.

Run ``python -m contextual_sparsity_mlp_amd.build``.  hipcc cross-compiles for
gfx950 without a GPU present.  The library lands in ``contextual_sparsity_mlp_amd/_lib``.
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
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libdv.so")
SOURCES = ["dv_api.hip", "dv_kernels.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code: the compiler would
# otherwise form v_pk_* fp32 ops from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile each source to an object in parallel, then link the shared library."""
    os.makedirs(LIBDIR, exist_ok=True)
    tag = f".tmp{os.getpid()}"
    common = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-Wno-unused-function", *DEVICE_FLAGS, "-I", INCLUDE]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(LIBDIR, os.path.splitext(src)[0] + tag + ".o")
        cmd = [*common, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                      text=True))
    failed = False
    for p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            failed = True
            sys.stderr.write(out + err)
        elif verbose and (out or err):
            sys.stderr.write(out + err)
    tmp = LIB + tag
    try:
        if failed:
            raise RuntimeError("hipcc failed to compile the sources")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
