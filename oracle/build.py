"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with g++.

-ffp-contract=off keeps every rounding exactly where the source writes it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "mxfp8_oracle.cpp")
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
