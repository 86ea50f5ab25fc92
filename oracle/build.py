"""Build the CPU oracle shared library (test infrastructure only).

Plain gcc, no fast-math and no floating-point contraction, so that every float
operation in the oracle is one IEEE-754 binary32 operation in source order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libw4oracle.so")
# Host sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer), loaded
# instead of LIB when W4_ORACLE_LIB names it; the process needs the gcc ASan
# runtime preloaded (LD_PRELOAD=$(gcc -print-file-name=libasan.so)).
LIB_SAN = os.path.join(HERE, "libw4oracle_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    src = os.path.join(HERE, "w4_oracle.c")
    out = LIB_SAN if sanitize else LIB
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-frounding-math", "-Wall", "-Wextra", "-Werror"]
    cmd += SAN_FLAGS if sanitize else []
    cmd += ["-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)
