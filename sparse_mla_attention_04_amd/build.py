"""Build the HIP/C++ library in-tree for gfx950.

    python -m sparse_mla_attention_04_amd.build

compiles csrc/*.cpp and csrc/*.hip with hipcc into
sparse_mla_attention_04_amd/lib/libsparse_mla.so (ahead of time: no JIT at run
time).  Packed fp32 instruction selection is disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libsparse_mla.so"
LIBPATH = os.path.join(LIBDIR, LIBNAME)
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".cpp", ".hip")))


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIBPATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include")] + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed (%d)" % r.returncode)
    os.replace(tmp, LIBPATH)
    return LIBPATH


if __name__ == "__main__":
    print(build(verbose=True))
