"""Build the plain-C CPU oracle (test infrastructure) into oracle/liboracle.so.

The oracle is compiled with gcc, OpenMP over rows, and -ffp-contract=off so that every
single-precision product and sum in the RoPE step is rounded on its own.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def command(src=SRC, out=LIB):
    return ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Wextra", src, "-o", out, "-lm"]


def build(verbose: bool = False) -> str:
    cmd = command(SRC, LIB + ".tmp")
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
