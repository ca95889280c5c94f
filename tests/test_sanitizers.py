"""Host code under the address and undefined-behaviour sanitizers (CPU only).

* The library's host code (argument checks, workspace layout, the C ABI
  surface) is compiled with the sanitizers on the host side only (device code
  unchanged), linked into a separate copy of libflowcache.so under the test's
  temporary directory, and driven by the C caller of test_abi_c.py; nothing
  is queued on a GPU.
* The C half of the oracle runs its pins (importance sums to one, closed-form
  redundancy equals the brute force, zero queries give uniform importance)
  on small inputs under the same sanitizers.
Any sanitizer report fails the test.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_compression_fc_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _clean(r):
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    return out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="hipcc or clang not available")
def test_library_host_code_under_sanitizers(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", *SAN_HOST, "-c", src, "-o", obj], check=True,
                       capture_output=True)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libflowcache.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *SAN_HOST, "-o", lib], check=True,
                   capture_output=True)
    exe = str(tmp_path / "abi_c")
    subprocess.run([CLANG, "-std=c99", "-Wall", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "native", "abi_c.c"),
                    "-L", str(tmp_path), "-lflowcache", "-Wl,-rpath," + str(tmp_path), "-o", exe], check=True)
    out = _clean(subprocess.run([exe], capture_output=True, text=True, timeout=120, env=ENV))
    assert "C ABI checks ok" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_c_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "native", "oracle_check.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe], check=True)
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=1")
    out = _clean(subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env))
    assert "oracle checks ok" in out
