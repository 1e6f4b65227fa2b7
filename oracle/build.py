"""Builds the CPU oracle (test infrastructure) with the host C++ compiler.

The oracle is plain C++17 compiled by g++; it never sees hipcc, the HIP
headers or any source of the GPU library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hpkv_oracle.cpp")
LIB = os.path.join(HERE, "liboracle_hpkv.so")


def build(verbose: bool = False) -> str:
    cxx = os.environ.get("CXX_ORACLE", "g++")
    tmp = LIB + ".tmp"
    cmd = [cxx, "-std=c++17", "-O2", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
