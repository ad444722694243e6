"""Build the CPU oracle shared library (test infrastructure only).

The oracle is plain C compiled with gcc, without -ffast-math (which would
flush denormals and license reassociation) and without FP contraction.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ar_oracle.c")
LIB = os.path.join(HERE, "libar_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile oracle/ar_oracle.c into oracle/libar_oracle.so; return its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
