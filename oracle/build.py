"""Compile the fp64 oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is built here so that tests can load it; building it is not
using it. -ffp-contract=off keeps every multiply and add a separately rounded IEEE operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


SAN_LIB = os.path.join(HERE, "liboracle_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build liboracle.so; with sanitize, liboracle_san.so instead: the same source under
    AddressSanitizer and UndefinedBehaviorSanitizer (any UB report aborts), for
    tests/test_sanitizers.py, which loads it into a Python that preloads gcc's ASan runtime."""
    src = os.path.join(HERE, "oracle.c")
    out = SAN_LIB if sanitize else LIB
    opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["gcc"] + opt + ["-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           "-fno-fast-math", "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
    sys.exit(0)
