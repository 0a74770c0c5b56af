"""Build the CPU oracle (oracle.c -> liboracle.so) with gcc.

Test infrastructure: the product library never links or loads it.
Strict IEEE evaluation (no -ffast-math), so every sum runs in index order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
