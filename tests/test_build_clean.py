"""The build entry point works from a clean checkout.

The built libraries are not committed, so a fresh clone holds no libhpkv.so.
This copies every file the repository would commit (tracked plus untracked,
not ignored) into an empty directory and runs ``__graft_entry__.build()``
there in a new interpreter: it must compile the HIP library and the oracle
and import the package, without any library built beforehand.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _committable_files():
    if shutil.which("git") is None or not os.path.isdir(os.path.join(ROOT, ".git")):
        pytest.skip("not a git checkout")
    r = subprocess.run(["git", "ls-files", "-z", "--cached", "--others", "--exclude-standard"],
                       cwd=ROOT, capture_output=True, check=True)
    return [f for f in r.stdout.decode().split("\0") if f]


def test_build_from_clean_checkout(tmp_path):
    if not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not installed")
    files = _committable_files()
    assert not any(f.endswith(".so") for f in files), "built libraries must not be committed"
    dst = tmp_path / "checkout"
    for f in files:
        src = os.path.join(ROOT, f)
        if not os.path.isfile(src):  # deleted in the working tree
            continue
        os.makedirs(os.path.dirname(dst / f), exist_ok=True)
        shutil.copy2(src, dst / f)
    lib = dst / "paged_kv_cache_hpkv_amd" / "libhpkv.so"
    assert not lib.exists()
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"],
                       cwd=dst, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert lib.exists()
    assert (dst / "oracle" / "liboracle_hpkv.so").exists()
    # a second import in a fresh process finds the library current and builds nothing
    r = subprocess.run([sys.executable, "-c", "import paged_kv_cache_hpkv_amd"], cwd=dst, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "building it with hipcc" not in r.stderr
