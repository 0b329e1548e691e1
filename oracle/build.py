"""Compile the fp64 oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is built here so that tests can load it; building it is not
using it. -ffp-contract=off keeps every multiply and add a separately rounded IEEE operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
