"""Compile the oracle's C file into oracle/liboracle.so with gcc.

The flags keep IEEE fp32 semantics: no fast-math, no FMA contraction, so every
operation in tq_oracle.c is rounded once in the order written. OpenMP only
splits independent vectors or rows across threads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
