"""gfx950 code generation of the library's own kernels, read from the assembly
hipcc writes for this repository's sources with the library's build flags
(CPU only; no GPU needed).

- y updates: the fp32 atomic adds compile to the hardware instruction
  (global_atomic_add_f32), never to a compare-and-swap loop on global memory;
  the ELL kernels, whose lanes own their rows, use no atomics at all.
- blocked COO sums into its LDS partials by compare-and-swap
  (ds_cmpst_rtn_b32), never by the LDS float atomic, which costs about seven
  times as much per wave instruction on gfx950.
- no packed-fp32 instructions anywhere: the build switches that code
  generation off.
"""
from __future__ import annotations

import collections
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from spmv_storage_formats_amd import _build

SOURCES = _build.sources() + [_build.BENCH_SRC]


def _kernels(asm: str) -> dict[str, str]:
    """Body of every function in an AMDGPU assembly file, by mangled name."""
    out, name = collections.defaultdict(list), None
    for line in asm.splitlines():
        m = re.match(r"\s*\.type\s+(\S+),@function", line)
        if m:
            name = m.group(1)
        elif line.startswith(".Lfunc_end"):
            name = None
        elif name:
            out[name].append(line)
    return {k: "\n".join(v) for k, v in out.items()}


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(_build.HIPCC):
        pytest.skip("hipcc not installed")
    d = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        out = d / (os.path.basename(src) + ".s")
        cmd = [_build.HIPCC, *_build.CFLAGS, "--cuda-device-only", "-S", src, "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return os.path.basename(src), _kernels(out.read_text())

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        per_file = dict(ex.map(compile_one, SOURCES))
    return per_file


def _find(kernels, file, stem):
    found = {k: v for k, v in kernels[file].items() if re.search(rf"\d{stem}[EI]", k)}
    assert found, (file, stem)
    return found


# kernels that add a sum into y
Y_ADDERS = ["k_coo_atomic", "k_coo_segmented", "k_csr_scalar", "k_csr_scalar_lds", "k_csr_vector",
            "k_jds", "k_sell", "k_merge", "k_merge_slices"]


@pytest.mark.parametrize("stem", Y_ADDERS)
def test_y_updates_are_hardware_fp32_atomics(kernels, stem):
    for name, body in _find(kernels, "spmv_kernels.hip", stem).items():
        assert "global_atomic_add_f32" in body, name
        assert "global_atomic_cmpswap" not in body, name


def test_blocked_coo_atomics(kernels):
    for name, body in _find(kernels, "coo_blocked.hip", "k_coo_blocked").items():
        assert "global_atomic_add_f32" in body, name
        assert "ds_cmpst_rtn_b32" in body, name
        assert not re.search(r"\bds_add(_rtn)?_f32\b", body), name
        assert "global_atomic_cmpswap" not in body, name


@pytest.mark.parametrize("stem", ["k_ell", "k_ell4", "k_ell_xtile"])
def test_ell_kernels_store_y_without_atomics(kernels, stem):
    for name, body in _find(kernels, "spmv_kernels.hip", stem).items():
        assert not re.search(r"\b(global|flat|buffer)_atomic_\w+", body), name
        assert re.search(r"\bglobal_store_dword", body), name


def test_no_global_cas_loops_anywhere(kernels):
    for file, ks in kernels.items():
        for name, body in ks.items():
            assert "global_atomic_cmpswap" not in body, (file, name)


def test_no_packed_fp32_instructions(kernels):
    pk = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
    n = 0
    for file, ks in kernels.items():
        for name, body in ks.items():
            assert not pk.search(body), (file, name)
            n += 1
    assert n > 40   # every kernel of the library and the microbenchmarks was read
