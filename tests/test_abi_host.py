"""C-ABI checks that need no GPU: the library loads, exports every function
include/spmv.h declares, and its host-only logic (the format selector, status
strings, argument checks that return before any device call) behaves."""
import ctypes

import numpy as np
import pytest

import oracle
import spmv_storage_formats_amd as spmv
from spmv_storage_formats_amd import synth


@pytest.fixture(scope="module")
def lib():
    return spmv.load_library()


def test_exports_every_declared_function(lib):
    names = spmv.declared_functions()
    assert len(names) >= 13
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_constants_match_the_header():
    """The binding's copies of the header's layout and limit constants."""
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(spmv.__file__), "..", "include", "spmv.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (SPMV_\w+) (\d+)", hdr)}
    assert defs["SPMV_BC_BLOCK_ROWS"] == spmv.BC_BLOCK_ROWS
    assert defs["SPMV_BC_BLOCK_ROWS_TALL"] == spmv.BC_BLOCK_ROWS_TALL
    assert spmv.BC_BLOCK_ROWS_TALL + 32 < 0xFFFF
    assert defs["SPMV_CG_NOALLOC_MAX_ROWS"] == spmv.CG_NOALLOC_MAX_ROWS
    assert spmv.BC_BLOCK_ROWS + 32 < 0xFFFF   # row codes and hot codes fit 16 bits


def test_library_is_gfx950_only():
    """The shared library carries a gfx950 code object and no other target."""
    data = open(spmv.library_path(), "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data
    for other in (b"--gfx942", b"--gfx90a", b"--gfx1100", b"sm_"):
        assert other not in data


def test_status_and_format_names(lib):
    assert lib.spmv_status_string(0) == b"ok"
    assert b"row pointers" in lib.spmv_status_string(2)
    for name, v in spmv.FORMATS.items():
        assert lib.spmv_format_name(v).decode() == name


def test_opts_default(lib):
    o = spmv._Opts()
    lib.spmv_opts_default(ctypes.byref(o))
    assert (o.hyb_width, o.lanes_per_row, o.validate, o.jds_depth, o.col_blocks, o.reserved,
            o.max_bytes) == (0, 0, 1, 0, 0, 0, 0)


def test_argument_checks_before_device(lib):
    out = ctypes.c_void_p(123)
    # null output handle / negative sizes / bad format / bad lanes: rejected on the host
    assert lib.spmv_build(None, 0, 4, 4, 8, None, None, None, None, None) == 1
    assert lib.spmv_build(ctypes.byref(out), 0, -1, 4, 8, None, None, None, None, None) == 1
    assert out.value is None
    assert lib.spmv_build(ctypes.byref(out), 42, 4, 4, 8, ctypes.c_void_p(8),
                          ctypes.c_void_p(8), ctypes.c_void_p(8), None, None) == 1
    o = spmv._opts(lanes=3)
    assert lib.spmv_build(ctypes.byref(out), 4, 4, 4, 8, ctypes.c_void_p(8), ctypes.c_void_p(8),
                          ctypes.c_void_p(8), ctypes.byref(o), None) == 1
    assert lib.spmv_run(None, None, None, None) == 1
    assert lib.spmv_destroy(None) == 0
    assert lib.spmv_get_info(None, None) == 1


def _stats(R, lens):
    lens = np.asarray(lens, np.int64)
    return {"num_rows": R, "num_cols": R, "nnz": int(lens.sum()), "max_len": int(lens.max()),
            "sum_len_sq": int((lens * lens).sum()), "empty_rows": int((lens == 0).sum()),
            "col_spread": 0}


def _hist(lens):
    return np.bincount(np.asarray(lens), minlength=int(np.max(lens)) + 1).astype(np.int64)


@pytest.mark.parametrize("case", range(60))
def test_selector_matches_oracle(case):
    """The library's selector and the oracle's (separately written) agree on
    random length distributions covering every branch."""
    rng = np.random.default_rng(9000 + case)
    R = int(rng.integers(1, 3000))
    kind = case % 5
    if kind == 0:
        lens = rng.integers(3, 7, size=R)                        # regular -> ELL
    elif kind == 1:
        lens = rng.integers(0, 4, size=R); lens[rng.integers(R)] = 60   # short + long -> COO
    elif kind == 2:
        lens = rng.integers(10, 21, size=R)
        lens[rng.choice(R, max(1, R // 200), replace=False)] = 1000  # HYB
    elif kind == 3:
        lens = np.floor(2.3 * (1 - rng.random(R)) ** (-1 / 1.1)).astype(np.int64)  # merge
    else:
        lens = rng.integers(8, 40, size=R)                       # CSR vector
    hw = int(rng.integers(0, 30)) if case % 7 == 0 else 0
    st = _stats(R, lens)
    h = _hist(lens)
    got = spmv.select(st, h, hyb_width=hw)
    exp = oracle.select(R, st["nnz"], h, hw)
    assert got == exp


@pytest.mark.parametrize("name", ["c1s", "c2s", "c3s", "c4s", "c5s", "fig14_1"])
def test_selector_on_workloads(name):
    w = synth.workload(name)
    st = oracle.row_stats(w.row_ptrs)
    stats = {"num_rows": w.num_rows, "num_cols": w.num_cols, "nnz": w.nnz, "max_len": st["W"],
             "sum_len_sq": st["sum_len_sq"], "empty_rows": st["empty_rows"], "col_spread": 0}
    assert spmv.select(stats, st["hist"]) == oracle.select(w.num_rows, w.nnz, st["hist"])
    expect = {"c1s": "ell", "c2s": "ell", "c3s": "ell", "c4s": "hyb", "c5s": "csr_merge",
              "fig14_1": "ell"}[name]
    assert spmv.select(stats, st["hist"])[0] == expect


def test_selector_skewed_full_gives_width_20():
    """The skewed workload (2M rows, 10-20 nnz + 50 long rows) selects HYB(20),
    the width the format-choice article (4.1) found best."""
    rng = np.random.default_rng(4)
    lens = rng.integers(10, 21, size=2_000_000)
    lens[rng.choice(2_000_000, 50, replace=False)] = rng.integers(1000, 5001, size=50)
    st = _stats(2_000_000, lens)
    assert spmv.select(st, _hist(lens)) == ("hyb", 20, 0)


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        spmv.build("ell", torch.zeros(5, dtype=torch.int32), torch.zeros(0, dtype=torch.int32),
                   torch.zeros(0), 4)


def test_selector_respects_int32_slots():
    """At the largest matrix the ABI accepts (nnz = INT32_MAX: 2^26 rows of 32,
    the last of 31) ELL would need 2^31 slots: both selectors fall through to
    CSR vector with 32 lanes.  A HYB choice whose ELL part exceeds int32 becomes
    merge-based CSR."""
    R = 2**26
    lens = np.full(R, 32, np.int64)
    lens[-1] = 31
    st = _stats(R, lens)
    assert st["nnz"] == 2**31 - 1
    h = _hist(lens)
    assert spmv.select(st, h) == ("csr_vector", 0, 32)
    assert oracle.select(R, st["nnz"], h) == ("csr_vector", 0, 32)
    # one row fewer: W*R = 2^31 - 32 fits, ELL
    st2 = _stats(R - 1, lens[:-1])
    assert spmv.select(st2, _hist(lens[:-1])) == ("ell", 0, 0)
    assert oracle.select(R - 1, st2["nnz"], _hist(lens[:-1])) == ("ell", 0, 0)
    # HYB: 2^26 rows of 20 plus 1000 rows of 150,000 (nnz ~1.49e9).  Forced width 33
    # passes the 1.5*nnz rule (2RK = 4.43e9 <= 3 nnz = 4.48e9) but R*K = 2.2e9 exceeds
    # int32 -> merge; width 31 fits both -> HYB.
    lens3 = np.full(R, 20, np.int64)
    lens3[:1000] = 150_000
    st3 = _stats(R, lens3)
    h3 = _hist(lens3)
    assert 2 * R * 33 <= 3 * st3["nnz"] and R * 33 > 2**31 - 1
    assert spmv.select(st3, h3, hyb_width=31) == ("hyb", 31, 0)
    assert oracle.select(R, st3["nnz"], h3, 31) == ("hyb", 31, 0)
    assert spmv.select(st3, h3, hyb_width=33) == ("csr_merge", 0, 0)
    assert oracle.select(R, st3["nnz"], h3, 33) == ("csr_merge", 0, 0)
