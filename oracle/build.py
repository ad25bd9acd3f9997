"""Build the fp64 CPU oracle (oracle.c) into liboracle.so next to this file.

Test infrastructure only: the product library never links or loads it.
Strict IEEE double arithmetic: no fast-math, no FMA contraction.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
        "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
