"""Build libw4a16.so for gfx950 with hipcc, in-tree.

    python -m bit_weight_only_w4a16_amd.build [--asm]

Compiles every csrc/*.hip and csrc/*.cpp to an object under _build/ (in
parallel) and links bit_weight_only_w4a16_amd/libw4a16.so.  Packed fp32
VALU instructions are disabled for all device code.  ``--asm`` also keeps the
gfx950 assembly of each translation unit under _build/asm/.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    "-I", os.path.join(ROOT, "include"),
]

# Per-file code generation options.  The split-K kernel holds its matrix
# accumulators in ordinary VGPRs (it fits in 256 of them at one wave per
# SIMD): with accumulation registers the compiler moves every accumulator
# out and back for each scale step (~350 extra moves per wave).
FILE_FLAGS = {
    "w4_splitk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, asm: bool) -> str:
    base = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(BUILD, base + ".o")
    extra = FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [hipcc()] + COMMON_FLAGS + extra + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    if asm:
        adir = os.path.join(BUILD, "asm")
        os.makedirs(adir, exist_ok=True)
        out = os.path.join(adir, base + ".s")
        cmd = ([hipcc()] + COMMON_FLAGS + extra +
               ["-x", "hip", "--cuda-device-only", "-S", src, "-o", out])
        subprocess.run(cmd, check=True, capture_output=True)
    return obj


def build(asm: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) +
                  glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built %s from %d sources" % (LIB, len(srcs)))
    return LIB


if __name__ == "__main__":
    build(asm="--asm" in sys.argv)
