"""Build libcdl.so (the HIP library) in-tree for gfx950.

    python -m combine_dispatch_layout_amd.build

Every HIP source is compiled with hipcc for gfx950 only.  Packed fp32 VALU
instructions are switched off (-packed-fp32-ops): the kernels only use scalar
fp32 arithmetic, and this keeps the compiler from fusing pairs of fp32 lanes
into v_pk_* forms.  hipcc's host pass prints that it does not know the
feature; that note is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(PKG, "csrc", "cdl.hip")]
LIB = os.path.join(PKG, "libcdl.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    "-I", INCLUDE,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile libcdl.so; always recompiles."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    if out.strip() and verbose:
        print(out, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
