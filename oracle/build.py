"""Builds the CPU oracle shared library (test infrastructure only).

    python oracle/build.py

Compiles microadam_oracle.c with gcc into liboracle_microadam.so next to this
file.  No fast-math, no floating-point contraction: the oracle's fp32
arithmetic is one rounding per operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "microadam_oracle.c")
LIB = os.path.join(HERE, "liboracle_microadam.so")

CFLAGS = ["-O2", "-std=gnu99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-strict-aliasing", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
