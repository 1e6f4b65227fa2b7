"""Builds libhpkv.so (the gfx950 HIP library behind include/hpkv.h) in-tree.

Every source is compiled by hipcc for gfx950 only; objects go to _build/ and
the shared library to paged_kv_cache_hpkv_amd/libhpkv.so. Packed fp32 VALU
instructions are disabled for all device code.

This file imports nothing from the package (the package loads the library at
import, so it cannot be imported before the library exists): run it as a
script, load it by file path, or import it as a submodule once built. Beside
the library it writes libhpkv.so.srchash, a digest of every source, header and
build flag; ``up_to_date()`` compares it with the tree so a loader can tell a
missing or stale library from a current one.
"""
import fcntl
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhpkv.so")
STAMP = LIB + ".srchash"
# (object name, source, extra defines): the decode source is compiled once per
# part so its kernel instantiations build in parallel
UNITS = [("hpkv_api", "hpkv_api.cpp", []),
         ("hpkv_slots_store", "hpkv_slots_store.hip", []),
         ("hpkv_decode_common", "hpkv_decode.hip", ["-DHPKV_DECODE_PART=0"]),
         ("hpkv_decode_f32", "hpkv_decode.hip", ["-DHPKV_DECODE_PART=1"]),
         ("hpkv_decode_f16", "hpkv_decode.hip", ["-DHPKV_DECODE_PART=2"]),
         ("hpkv_decode_bf16", "hpkv_decode.hip", ["-DHPKV_DECODE_PART=3"]),
         ("hpkv_decode_quant_f32", "hpkv_decode.hip", ["-DHPKV_DECODE_PART=4"]),
         ("hpkv_decode_quant_f16", "hpkv_decode.hip", ["-DHPKV_DECODE_PART=5"]),
         ("hpkv_decode_quant_bf16", "hpkv_decode.hip", ["-DHPKV_DECODE_PART=6"]),
         ("hpkv_prefill", "hpkv_prefill.hip", []),
         ("hpkv_ceiling", "hpkv_ceiling.hip", []),
         ("hpkv_noalloc", "hpkv_noalloc.hip", []),
         ("hpkv_blocks", "hpkv_blocks.cpp", [])]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def source_hash() -> str:
    """Digest of every file the library is built from plus the build flags."""
    h = hashlib.sha256()
    h.update(repr((HIPCC, COMMON, UNITS)).encode())
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".cpp", ".h")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    with open(os.path.abspath(__file__), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def up_to_date() -> bool:
    if not (os.path.exists(LIB) and os.path.exists(STAMP)):
        return False
    with open(STAMP) as f:
        return f.read().strip() == source_hash()


def _compile(unit, verbose):
    name, src, defs = unit
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + defs + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {' '.join(defs)}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    print(f"[hpkv build] compiled {name}", file=sys.stderr, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every unit and links libhpkv.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with open(os.path.join(BUILD, "libhpkv.lock"), "w") as lock:
        fcntl.flock(lock, fcntl.LOCK_EX)
        digest = source_hash()
        workers = max(1, min(len(UNITS), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            objs = list(ex.map(lambda u: _compile(u, verbose), UNITS))
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
        with open(STAMP + ".tmp", "w") as f:
            f.write(digest + "\n")
        os.replace(STAMP + ".tmp", STAMP)
    return LIB


def ensure_built() -> str:
    """Builds the library only when it is missing or older than its sources."""
    if not up_to_date():
        os.makedirs(BUILD, exist_ok=True)
        with open(os.path.join(BUILD, "libhpkv.ensure.lock"), "w") as lock:
            fcntl.flock(lock, fcntl.LOCK_EX)
            if not up_to_date():  # another process may have built it meanwhile
                print("[hpkv build] libhpkv.so missing or stale: building it with hipcc",
                      file=sys.stderr, flush=True)
                build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
