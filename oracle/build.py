"""Compile the CPU oracle (``sgemm_oracle.c``) into ``liboracle.so`` with gcc.

Test infrastructure only.  Plain gcc, no BLAS, no fast-math, no FMA
contraction, so the fp64 arithmetic is exactly what the C source says.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sgemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(verbose: bool = False) -> str:
    """Build liboracle.so next to the source; returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
