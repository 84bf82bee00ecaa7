"""Build the fp64 CPU oracle (test infrastructure) with gcc + OpenMP.

Usage: python oracle/build.py      (writes oracle/liboracle.so)
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "flux_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = True) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
