"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, fp64, no fast-math and no FMA contraction, OpenMP over independent
rows only.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-D_GNU_SOURCE", "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra=(), cc="gcc", openmp=True):
    """Compile `src` to the shared library `out` with `cc`; returns `out`."""
    flags = [f for f in CFLAGS if openmp or f != "-fopenmp"]
    cmd = [cc, *flags, *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
