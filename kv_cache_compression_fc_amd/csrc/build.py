"""Build libflowcache.so for gfx950 with hipcc (in-tree).

Each ``*.hip`` file under ``csrc/`` is compiled to an object in
``csrc/_build/`` and linked into ``kv_cache_compression_fc_amd/libflowcache.so``.
Packed-fp32 instructions are disabled for the device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(PKG, "libflowcache.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into VGPRs (no v_accvgpr_read per element)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(HERE, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


MICROBENCH = os.path.join(HERE, "microbench")


def build_microbench(verbose: bool = False) -> list:
    """Stand-alone measurement programs (not part of the library): each
    ``microbench/*.hip`` becomes an executable in ``csrc/_build/``."""
    os.makedirs(BUILD, exist_ok=True)
    exes = []
    for src in sorted(glob.glob(os.path.join(MICROBENCH, "*.hip"))):
        exe = os.path.join(BUILD, os.path.basename(src)[:-4])
        cmd = [HIPCC, *[f for f in CFLAGS if f != "-fPIC"], src, "-o", exe]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        exes.append(exe)
    return exes


if __name__ == "__main__":
    build(verbose=True)
    build_microbench(verbose=True)
