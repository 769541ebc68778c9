"""Build the C-ABI library ``_lib/libppa.so`` in-tree with hipcc for gfx950.

Usage: ``python paged_kv_prefill_varlen_amd/build.py`` (or ``__graft_entry__.build()``).
It is run as a script because importing the package needs the built library.
The host validator is plain C++ and the kernels are HIP; both go into one
shared library.  Packed FP32 instructions are disabled for the device code.
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
LIB = os.path.join(LIBDIR, "libppa.so")
ARCH = os.environ.get("PPA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["ppa_host.cpp", "ppa_attention.hip", "ppa_validate.hip"]
HEADERS = ["ppa_internal.h", "ppa_page_addr.hpp"]

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library.  Always rebuilds."""
    os.makedirs(LIBDIR, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    tmpdir = os.path.join(LIBDIR, "obj")
    os.makedirs(tmpdir, exist_ok=True)
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(tmpdir, src + ".o")
        if src.endswith(".hip"):
            cmd = [hipcc, *DEVICE_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", path, "-o", obj]
        else:
            # host-only translation unit: no device code, no offload
            cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-x", "c++", "-I", INCLUDE, "-I", CSRC,
                   "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
