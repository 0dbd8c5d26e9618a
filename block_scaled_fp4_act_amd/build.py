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
SOURCES = ["api.cpp", "quant.hip", "prepack.hip", "calib.hip", "gemm.hip", "gemm_tile.hip", "gemm_tile_dma.hip", "attn.hip", "scratch.hip", "stream_read.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source additions.  The attention kernel at D = 256 holds about 250
# registers; in the MFMA's default form the compiler parks values in AGPRs and
# copies them back and forth (a third of the loop's VALU instructions); in
# VGPR form it copies a fifth as much and the D = 256 decode step is 5-6 %
# faster (D = 128 is unchanged).  The tiled linear keeps the default form: its
# large tiles spill in VGPR form.
FILE_FLAGS = {
    "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def build(verbose=False, jobs=4):
    """Compile each source to an object (in parallel), then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cflags = [f for f in FLAGS if f != "-shared"]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + cflags + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
