"""Builds the reference oracle (plain C, double precision) into oracle/liboracle.so.

Test infrastructure only: the product path never loads this library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
