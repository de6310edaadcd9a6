"""Build the fp64 CPU oracle (oracle/liboracle.so) with gcc.

Test infrastructure only: the oracle checks the HIP library and is never part
of it.  Run `python oracle/build.py` or call `build()`.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "la_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
