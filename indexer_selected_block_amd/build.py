"""Builds libisb.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libisb.so")
# measurement kernels for the benchmark (include/isb_ceiling.h): not part of the layer
CEILING_LIB_PATH = os.path.join(PKG_DIR, "libisb_ceiling.so")

SOURCES = ["capi.hip", "index_score.hip", "topk_select.hip", "emit.hip", "sparse_pa.hip", "writer.hip", "merge.hip"]
CEILING_SOURCES = ["ceiling.hip"]

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


def _compile(sources, out_path, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out_path + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, out_path)
    return out_path


def build_library(verbose: bool = False) -> str:
    """Compile every kernel source into libisb.so next to this file; returns its path."""
    return _compile(SOURCES, LIB_PATH, verbose)


def build_ceiling_library(verbose: bool = False) -> str:
    """Compile the benchmark's measurement kernels into libisb_ceiling.so."""
    return _compile(CEILING_SOURCES, CEILING_LIB_PATH, verbose)


_MFMA = re.compile(r"^\s*(v_mfma\S*)\s+(.*)$")


def _reg_range(tok: str):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return m.group(1), int(m.group(2)), int(m.group(3))
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return m.group(1), int(m.group(2)), int(m.group(2))
    return None


def mfma_operand_overlaps(asm: str) -> list:
    """MFMA instructions of gfx950 assembly whose destination registers overlap
    a source operand other than an identical accumulator (the register
    allocator has placed the scaled fp4 MFMA's destination over a source,
    which corrupts the product)."""
    bad = []
    for line in asm.splitlines():
        m = _MFMA.match(line)
        if not m:
            continue
        ops = [o.strip() for o in m.group(2).split(",")]
        d = _reg_range(ops[0])
        for k, src in enumerate(_reg_range(o) for o in ops[1:4]):
            if not d or not src or src[0] != d[0]:
                continue
            overlap = not (src[2] < d[1] or src[1] > d[2])
            if overlap and not (k == 2 and src[1:] == d[1:]):
                bad.append(line.strip())
    return bad


def check_mfma_operands() -> int:
    """Compiles every source to gfx950 assembly and raises if any MFMA
    destination overlaps a source; returns the number of MFMAs checked."""
    total = 0
    with tempfile.TemporaryDirectory() as tmp:
        for src in SOURCES:
            out = os.path.join(tmp, src + ".s")
            flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
            cmd = [hipcc(), *flags, "--cuda-device-only", "-S", "-I", INCLUDE, "-I", CSRC,
                   os.path.join(CSRC, src), "-o", out]
            proc = subprocess.run(cmd, capture_output=True, text=True)
            if proc.returncode != 0:
                raise RuntimeError(f"hipcc -S {src} failed ({proc.returncode}):\n{proc.stderr}")
            asm = open(out).read()
            total += sum(1 for line in asm.splitlines() if _MFMA.match(line))
            bad = mfma_operand_overlaps(asm)
            if bad:
                raise RuntimeError(f"{src}: MFMA destination overlaps a source:\n" + "\n".join(bad[:10]))
    return total


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_ceiling_library(verbose=True))
    print(f"checked {check_mfma_operands()} MFMA instructions: no operand overlap")
