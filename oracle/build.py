"""Compile the CPU oracle (plain C, double precision) into oracle/liboasis_oracle.so.

Test infrastructure: building the checker is not using it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboasis_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
