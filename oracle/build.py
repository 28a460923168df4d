"""Builds the oracle's C core (``attention.c``) into ``liboracle.so`` with gcc.

Test infrastructure: the library this writes is loaded only by the tests,
the smoke check and the CPU-baseline leg of the benchmark.

Plain ``-O2`` and no ``-ffast-math``: the compiler may not reassociate the
fp64 sums, so every row is summed exactly in the order the source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attention.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    """Returns the library path, compiling first only if nothing is built."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
