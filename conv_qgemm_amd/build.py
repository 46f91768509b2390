"""Build libqgemm.so in-tree with hipcc for gfx950 (CDNA4 / MI355X).

The library's HIP sources under ``csrc/`` are compiled to objects in
parallel and linked into ``conv_qgemm_amd/libqgemm.so``; the benchmark's
calibration kernels (``csrc/calib.hip``) go to their own
``conv_qgemm_amd/libqgcalib.so``.  Objects go to ``_build/`` at the
repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "qgemm")
LIB = os.path.join(PKG, "libqgemm.so")
CALIB_LIB = os.path.join(PKG, "libqgcalib.so")
CALIB_SOURCES = ["calib.hip"]
# the benchmark's comparison with AMD's hipBLASLt int8 GEMM (its own library,
# so that libqgemm.so does not depend on hipBLASLt)
VENDOR_LIB = os.path.join(PKG, "libqgvendor.so")
VENDOR_SOURCES = ["vendor_hipblaslt.cpp"]
SOURCES = ["api.cpp", "k_tile_gemm.hip", "k_gemm_dma.hip", "k_skinny_w4a8.hip", "k_conv_halo.hip", "k_dwconv.hip",
           "k_quant.hip", "k_zp.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-mcode-object-version=5",
    # no packed-fp32 instruction selection
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Per-source additions.  The large-GEMM ring keeps its 256 accumulators of
# 16x16 MFMA tiles in place only when the pre-RA machine scheduler is off:
# with it, the compiler reorders the loop's MFMAs so that about half of them
# write a different register quad than they read, and every K stage then
# pays 130-230 accumulator copies (measured in the generated code, and in the
# kernel: the matrix pipe busy 54% instead of 65%).  The loop's source order
# is already the intended schedule.
SRC_FLAGS = {
    "k_gemm_dma.hip": ["-mllvm", "-enable-misched=0"],
}


def flags_for(src: str):
    """Compiler flags of one source file under csrc/."""
    return [*CFLAGS, *SRC_FLAGS.get(os.path.basename(src), [])]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib, verbose, libs=()):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           "-Wl,-rpath,/opt/rocm/lib", *libs]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}", file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES + VENDOR_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    n, c = len(SOURCES), len(CALIB_SOURCES)
    _link(objs[:n], LIB, verbose)
    _link(objs[n:n + c], CALIB_LIB, verbose)
    _link(objs[n + c:], VENDOR_LIB, verbose, libs=["-L/opt/rocm/lib", "-lhipblaslt"])
    return LIB


if __name__ == "__main__":
    build(verbose=True)
