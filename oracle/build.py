"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, no GPU toolchain: -O2 without fast-math and with floating-point
contraction off, so every operation in kvq_oracle.c is one IEEE operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(extra_flags=(), out=LIB, verbose=False):
    """Compile the oracle; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *extra_flags, SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
