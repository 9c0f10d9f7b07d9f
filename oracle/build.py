"""Build the CPU oracle library (liboracle.so) with gcc.

Flags: no fast-math and no FMA contraction, so every double operation is the
IEEE operation written in oracle.c, on any x86-64 host; -fopenmp for the row
loops. Usage: ``python oracle/build.py``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-fno-strict-aliasing",
           "-Wall", "-Wextra", "-Wno-unused-parameter",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
