"""Build the CPU oracle shared library (test infrastructure only).

Plain gcc, no fast-math and no floating-point contraction, so that every float
operation in the oracle is one IEEE-754 binary32 operation in source order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libw4oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "w4_oracle.c")
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-frounding-math", "-Wall", "-Wextra", "-Werror",
           "-o", LIB + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
