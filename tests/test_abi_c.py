"""The C ABI from C: include/flowcache.h compiles as C99 with warnings as
errors, a C program links against libflowcache.so and its host-side checks
answer as documented (no GPU needed; nothing is queued)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "abi_c.c")
PKG = os.path.join(ROOT, "kv_cache_compression_fc_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_caller(tmp_path):
    from conftest import ensure_library
    ensure_library()
    exe = str(tmp_path / "abi_c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    SRC, "-L", PKG, "-lflowcache", "-Wl,-rpath," + PKG, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI checks ok" in r.stdout
