"""Compile the HIP library (libgdr.so) for gfx950 with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgdr.so")
SOURCES = [os.path.join(PKG, "csrc", n) for n in ("gdr_api.cpp", "gdr_kernels.hip", "gdr_chain.hip", "gdr_kda.hip", "gdr_out.hip", "gdr_group.hip", "gdr_tables.hip", "gdr_noalloc.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed-fp32 instructions stay off (hipcc would otherwise form v_pk_* from float2 code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out_tmp = LIB + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", out_tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgdr.so")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
