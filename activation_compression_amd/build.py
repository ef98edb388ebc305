"""Build the HIP library (libcoat.so) in-tree for gfx950.

hipcc cross-compiles without a GPU.  FP contraction is off so every FMA in
the kernels is one written explicitly; packed-FP32 instruction selection is
disabled (the kernels are scalar FP32 by design).
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcoat.so")
ARCH = os.environ.get("COAT_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc(out, srcs, verbose, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-o", out + ".tmp", *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, extra=()) -> str:
    _hipcc(LIB, sources(), verbose, extra)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
