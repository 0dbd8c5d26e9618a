"""Build step of the HIP library: compiles csrc/ into librsfp4.so for gfx950.

Every step of the path runs in these kernels; the Python package only loads
the result.  Flags: no FP contraction (the quantizer's s~ * e and x - d must
round separately), no fast-math, correctly rounded fp32 division (clang's HIP
default), and no packed-FP32 instruction selection.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librsfp4.so")
SOURCES = ["api.cpp", "quant.hip", "prepack.hip", "calib.hip", "gemm.hip", "gemm_tile.hip", "attn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
