"""Build the oracle's shared library with g++ (test infrastructure only).

Plain C++17, -O2, no fast-math, so every fp64 product and sum is evaluated in
source order.  Nothing from the HIP library is compiled or linked here.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-pthread", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
