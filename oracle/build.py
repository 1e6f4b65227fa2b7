"""Builds the CPU oracle (test infrastructure) with the host C++ compiler.

The oracle is plain C++17 compiled by g++; it never sees hipcc, the HIP
headers or any source of the GPU library. Beside the library it writes a
digest of the source and flags, so ``ensure_built()`` rebuilds a stale one.
"""
import fcntl
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hpkv_oracle.cpp")
LIB = os.path.join(HERE, "liboracle_hpkv.so")
STAMP = LIB + ".srchash"


def _cmd(out):
    cxx = os.environ.get("CXX_ORACLE", "g++")
    return [cxx, "-std=c++17", "-O2", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
            "-fno-fast-math", "-ffp-contract=off", SRC, "-o", out]


def source_hash() -> str:
    h = hashlib.sha256(repr(_cmd("")).encode())
    for path in (SRC, os.path.abspath(__file__)):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def up_to_date() -> bool:
    if not (os.path.exists(LIB) and os.path.exists(STAMP)):
        return False
    with open(STAMP) as f:
        return f.read().strip() == source_hash()


def build(verbose: bool = False) -> str:
    with open(os.path.join(HERE, ".build.lock"), "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        digest = source_hash()
        tmp = LIB + ".tmp"
        cmd = _cmd(tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
        with open(STAMP + ".tmp", "w") as f:
            f.write(digest + "\n")
        os.replace(STAMP + ".tmp", STAMP)
    return LIB


def ensure_built() -> str:
    if not up_to_date():
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
