"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with g++.

-ffp-contract=off keeps every rounding exactly where the source writes it.

build(sanitize=True) builds a second copy, oracle/liboracle_asan.so, with
AddressSanitizer and UndefinedBehaviorSanitizer (g++ only: the oracle is host
code).  The test suite loads it through MXFP8_ORACLE_LIB in a child process
that preloads the sanitizer runtime, and runs the oracle pins against it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
ASAN_LIB = os.path.join(HERE, "liboracle_asan.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    src = os.path.join(HERE, "mxfp8_oracle.cpp")
    out = ASAN_LIB if sanitize else LIB
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra"]
    if sanitize:
        cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    cmd += ["-o", out + ".tmp", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)
