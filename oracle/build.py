"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain C compiled with gcc; strict IEEE binary64 (no fast-math, no FMA
contraction) so that the oracle's arithmetic is exactly what the source says.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "coat_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off", "-fno-strict-aliasing",
         "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *FLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
