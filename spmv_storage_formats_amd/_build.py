"""Build the gfx950 HIP library ``libspmv_mi355x.so`` in the package directory.

Usage: ``python -m spmv_storage_formats_amd._build`` (or ``build()`` from
``__graft_entry__``).  Every .hip file under csrc/ is compiled for gfx950 only,
then linked into one shared library exporting the C ABI of include/spmv.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspmv_mi355x.so")
OBJDIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # hardware fp32 atomics (global_atomic_add_f32 / ds_add_f32), no CAS loops
    "-munsafe-fp-atomics",
    # no packed-fp32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


BENCH_SRC = os.path.join(PKG, "bench_csrc", "microbench.hip")
BENCH_LIB = os.path.join(PKG, "libspmv_microbench.so")


def build_microbench(verbose: bool = True) -> str:
    """The benchmark's gather / LDS-update microbenchmarks (not the library)."""
    tmp = BENCH_LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *CFLAGS, "-shared", BENCH_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {BENCH_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, BENCH_LIB)
    if verbose:
        print(f"built {BENCH_LIB}", file=sys.stderr)
    return BENCH_LIB


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link the library.  Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
    build_microbench()
