"""Builds libisb.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libisb.so")

SOURCES = ["capi.hip", "index_score.hip", "topk_select.hip", "emit.hip", "sparse_pa.hip"]

# gfx950 only.  Packed fp32 VALU ops are disabled (-packed-fp32-ops): the
# compiler must not form v_pk_{add,mul,fma}_f32 on its own.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build_library(verbose: bool = False) -> str:
    """Compile every kernel source into libisb.so next to this file; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
