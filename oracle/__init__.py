"""CPU oracle for y <- A*x + y (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The arithmetic lives in ``oracle.c`` (plain single-threaded C, fp64
accumulation); this module only marshals numpy arrays to it.  It shares no code
with the GPU library, and the GPU library never calls it.

Parity unpinned: none.  Every function here is pinned by tests that do not
re-use it (the printed worked examples of the pages, closed forms, dense
brute force); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_OMP_SRC = os.path.join(_HERE, "csr_omp.c")
_OMP_LIB = os.path.join(_HERE, "libcsr_omp.so")
_omp = None
_lock = threading.Lock()
_lib = None

OK, ERR_INVALID_ARG, ERR_BAD_ROWPTRS, ERR_BAD_COLIDX, ERR_BAD_ROWIDX, ERR_TOO_LARGE = range(6)
FMT_NAMES = {1: "coo_atomic", 2: "coo_segmented", 3: "csr_scalar", 4: "csr_vector",
             5: "ell", 6: "hyb", 7: "jds", 8: "csr_merge", 9: "sell", 10: "ell_xtile",
             11: "coo_blocked"}
RTOL = 1e-5

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, no fast-math, no FMA contraction)
    and the OpenMP CSR baseline csr_omp.c into libcsr_omp.so."""
    with _lock:
        if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            tmp = _LIB + f".tmp{os.getpid()}"
            subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                                   "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
            os.replace(tmp, _LIB)
        if (force or not os.path.exists(_OMP_LIB)
                or os.path.getmtime(_OMP_LIB) < os.path.getmtime(_OMP_SRC)):
            tmp = _OMP_LIB + f".tmp{os.getpid()}"
            subprocess.check_call(["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                                   "-ffp-contract=off", "-fno-fast-math", _OMP_SRC, "-o", tmp])
            os.replace(tmp, _OMP_LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    sig = {
        "orc_validate_csr": (ctypes.c_int, [_i64, _i64, _i64, _i32p, ctypes.c_void_p]),
        "orc_validate_coo": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_void_p, ctypes.c_void_p]),
        "orc_spmv_csr": (None, [_i64, _i32p, _i32p, _f32p, _f32p, _f32p, _f64p, _f64p]),
        "orc_spmv_coo": (None, [_i64, _i64, _i32p, _i32p, _f32p, _f32p, _f32p, _f64p, _f64p]),
        "orc_check": (_i64, [_i64, _f32p, _f64p, _f64p, ctypes.c_double,
                             ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double)]),
        "orc_coo_to_csr": (ctypes.c_int, [_i64, _i64, _i32p, _i32p, _u32p, _i32p, _i32p, _u32p]),
        "orc_csr_to_coo": (None, [_i64, _i32p, _i32p]),
        "orc_row_stats": (None, [_i64, _i32p, _i64p]),
        "orc_len_hist": (None, [_i64, _i32p, _i64, _i64p]),
        "orc_hyb_tail_count": (_i64, [_i64, _i32p, _i64]),
        "orc_csr_to_hyb": (ctypes.c_int, [_i64, _i32p, _i32p, _u32p, _i64, _i32p, _u32p, _i32p,
                                          _i32p, _i32p, _u32p]),
        "orc_csr_to_jds": (ctypes.c_int, [_i64, _i32p, _i32p, _u32p, _i64, _i32p, _i32p, _i32p,
                                          _i32p, _u32p]),
        "orc_sell_slots": (_i64, [_i64, _i32p, _i64]),
        "orc_csr_to_sell": (ctypes.c_int, [_i64, _i32p, _i32p, _u32p, _i64, _i32p, _i32p, _i32p,
                                           _i32p, _u32p]),
        "orc_hyb_width": (_i64, [_i64, _i64, _i64p]),
        "orc_vector_lanes": (_i64, [_i64, _i64]),
        "orc_select": (None, [_i64, _i64, _i64, _i64p, _i64, _i64, _i64p]),
        "orc_cg": (ctypes.c_int, [_i64, _i32p, _i32p, _f32p, _f64p, _f64p, _i64,
                                  ctypes.c_double, _f64p]),
        "orc_csr_to_ell_xtile": (ctypes.c_int, [_i64, _i32p, _i32p, _u32p, _i64, _i64,
                                                ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.POINTER(_i64)]),
        "orc_coo_blocked": (ctypes.c_int, [_i64, _i64, _i64, _i32p, _i32p, _u32p, _i64, _i64,
                                           _i64, _i64, _i64, _i64p] + [ctypes.c_void_p] * 10),
        "orc_select_build": (ctypes.c_int, [_i64, _i64, _i64, _i32p, _i32p, _i64, _i64p]),
        "orc_bc_chunk_entries": (_i64, [_i64]),
        "orc_bc_block_rows": (_i64, [_i64, _i64, _i64, _i32p, _i32p, _i64, _i64, _i64, _i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _bits(a):
    """fp32 array viewed as its raw uint32 bit patterns (builders move bits)."""
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _ptr_or_none(a):
    return None if a is None or a.size == 0 else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- validation

def validate_csr(num_rows, num_cols, row_ptrs, col_idx) -> int:
    rp, ci = _i32(row_ptrs), _i32(col_idx)
    if rp.shape[0] != num_rows + 1:
        return ERR_INVALID_ARG
    return int(_load().orc_validate_csr(num_rows, num_cols, ci.shape[0], rp, _ptr_or_none(ci)))


def validate_coo(num_rows, num_cols, row_idx, col_idx) -> int:
    ri, ci = _i32(row_idx), _i32(col_idx)
    if ri.shape != ci.shape:
        return ERR_INVALID_ARG
    return int(_load().orc_validate_coo(num_rows, num_cols, ci.shape[0], _ptr_or_none(ri),
                                        _ptr_or_none(ci)))


# ---------------------------------------------------------------------- SpMV

def spmv_csr(row_ptrs, col_idx, values, x, y):
    """Return (y_ref fp64, bound fp64) for y + A x with A in CSR."""
    rp = _i32(row_ptrs)
    R = rp.shape[0] - 1
    y_ref = np.empty(R, np.float64)
    bound = np.empty(R, np.float64)
    _load().orc_spmv_csr(R, rp, _i32(col_idx), _f32(values), _f32(x), _f32(y), y_ref, bound)
    return y_ref, bound


def spmv_coo(num_rows, row_idx, col_idx, values, x, y):
    y_ref = np.empty(num_rows, np.float64)
    bound = np.empty(num_rows, np.float64)
    ci = _i32(col_idx)
    _load().orc_spmv_coo(num_rows, ci.shape[0], _i32(row_idx), ci, _f32(values), _f32(x),
                         _f32(y), y_ref, bound)
    return y_ref, bound


def check(y_gpu, y_ref, bound, rtol: float = RTOL):
    """Row-wise bound |y_gpu - y_ref| <= rtol * bound.  Returns (n_bad, first_bad, worst)."""
    yg = _f32(y_gpu)
    first = _i64(-1)
    worst = ctypes.c_double(0.0)
    n = _load().orc_check(yg.shape[0], yg, np.ascontiguousarray(y_ref, np.float64),
                          np.ascontiguousarray(bound, np.float64), rtol,
                          ctypes.byref(first), ctypes.byref(worst))
    return int(n), int(first.value), float(worst.value)


# ------------------------------------------------------------------ builders

def coo_to_csr(num_rows, row_idx, col_idx, values):
    ri, ci, v = _i32(row_idx), _i32(col_idx), _bits(values)
    nnz = ci.shape[0]
    rp = np.empty(num_rows + 1, np.int32)
    oc = np.empty(nnz, np.int32)
    ov = np.empty(nnz, np.uint32)
    _load().orc_coo_to_csr(num_rows, nnz, ri, ci, v, rp, oc, ov)
    return rp, oc, ov.view(np.float32)


def csr_to_coo(row_ptrs):
    rp = _i32(row_ptrs)
    ri = np.empty(int(rp[-1]), np.int32)
    _load().orc_csr_to_coo(rp.shape[0] - 1, rp, ri)
    return ri


def row_stats(row_ptrs):
    """dict(W, nnz, sum_len_sq, empty_rows, hist) of the row lengths."""
    rp = _i32(row_ptrs)
    R = rp.shape[0] - 1
    out = np.zeros(4, np.int64)
    _load().orc_row_stats(R, rp, out)
    W = int(out[0])
    hist = np.zeros(W + 1, np.int64)
    _load().orc_len_hist(R, rp, W, hist)
    return {"W": W, "nnz": int(out[1]), "sum_len_sq": int(out[2]),
            "empty_rows": int(out[3]), "hist": hist}


def csr_to_hyb(row_ptrs, col_idx, values, K):
    """HYB(K): ELL part of width min(K, W) column-major + COO tail.

    Returns dict(width, ell_col, ell_val, ell_nnz, tail_row, tail_col, tail_val)
    or raises ValueError("too large") when R*width exceeds int32 range.
    """
    rp = _i32(row_ptrs)
    R = rp.shape[0] - 1
    W = row_stats(rp)["W"]
    Kw = min(int(K), W)
    if R * Kw > 2**31 - 1:
        raise ValueError("too large")
    lib = _load()
    ntail = int(lib.orc_hyb_tail_count(R, rp, Kw))
    ell_col = np.empty(R * Kw, np.int32)
    ell_val = np.empty(R * Kw, np.uint32)
    ell_nnz = np.empty(R, np.int32)
    tr = np.empty(ntail, np.int32)
    tc = np.empty(ntail, np.int32)
    tv = np.empty(ntail, np.uint32)
    st = lib.orc_csr_to_hyb(R, rp, _i32(col_idx), _bits(values), Kw, ell_col, ell_val,
                            ell_nnz, tr, tc, tv)
    if st == ERR_TOO_LARGE:
        raise ValueError("too large")
    return {"width": Kw, "ell_col": ell_col, "ell_val": ell_val.view(np.float32),
            "ell_nnz": ell_nnz, "tail_row": tr, "tail_col": tc,
            "tail_val": tv.view(np.float32)}


def csr_to_ell(row_ptrs, col_idx, values):
    """ELL: width W = longest row; same arrays as HYB with an empty tail."""
    W = row_stats(row_ptrs)["W"]
    h = csr_to_hyb(row_ptrs, col_idx, values, W)
    assert h["tail_row"].size == 0
    return {"width": h["width"], "col": h["ell_col"], "val": h["ell_val"], "nnz": h["ell_nnz"]}


def csr_to_jds(row_ptrs, col_idx, values):
    rp = _i32(row_ptrs)
    R = rp.shape[0] - 1
    W = row_stats(rp)["W"]
    nnz = int(rp[-1])
    perm = np.empty(R, np.int32)
    jlen = np.empty(R, np.int32)
    iptr = np.empty(W + 1, np.int32)
    jc = np.empty(nnz, np.int32)
    jv = np.empty(nnz, np.uint32)
    _load().orc_csr_to_jds(R, rp, _i32(col_idx), _bits(values), W, perm, jlen, iptr, jc, jv)
    return {"perm": perm, "len": jlen, "iter_ptr": iptr, "col": jc, "val": jv.view(np.float32)}


def csr_to_ell_xtile(row_ptrs, col_idx, values, block_rows=256):
    """ELL with x tiles: run_ptr, runs (k x 3: first column, tile offset, length),
    lidx (int16, column-major slots), val, nnz.  ValueError("too large") when refused."""
    rp = _i32(row_ptrs)
    R = rp.shape[0] - 1
    ci = _i32(col_idx)
    vb = _bits(values)
    W = int(np.diff(rp.astype(np.int64)).max()) if R > 0 else 0
    lib = _load()
    total = _i64(0)
    st = lib.orc_csr_to_ell_xtile(R, rp, ci, vb, W, block_rows, None, None, None, None, None,
                                  ctypes.byref(total))
    if st == ERR_TOO_LARGE:
        raise ValueError("too large")
    nb = (R + block_rows - 1) // block_rows
    run_ptr = np.zeros(nb + 1, np.int32)
    runs = np.zeros(3 * max(total.value, 1), np.int32)
    lidx = np.zeros(max(R * W, 1), np.int16)
    val = np.zeros(max(R * W, 1), np.uint32)
    nnz = np.zeros(max(R, 1), np.int32)
    st = lib.orc_csr_to_ell_xtile(R, rp, ci, vb, W, block_rows, run_ptr.ctypes.data,
                                  runs.ctypes.data, lidx.ctypes.data, val.ctypes.data,
                                  nnz.ctypes.data, ctypes.byref(total))
    assert st == OK
    return {"run_ptr": run_ptr, "runs": runs[:3 * total.value].reshape(-1, 3),
            "lidx": lidx[:R * W], "val": val[:R * W].view(np.float32), "nnz": nnz[:R],
            "width": W, "block_rows": block_rows}


def csr_to_coo_blocked(row_ptrs, col_idx, values, num_cols, slices, block_rows, chunk_entries,
                       hot_slots, hot_min_len):
    """Blocked COO: the arrays chunk_grp, chunk_blk, slice_chunk, slice_item, item_chunk,
    hot, base, pk (uint32), val (fp32 bit copies) and wide, as oracle.c defines them."""
    rp = _i32(row_ptrs)
    R = rp.shape[0] - 1
    ci = _i32(col_idx)
    vb = _bits(values)
    nnz = ci.shape[0]
    lib = _load()
    sizes = np.zeros(5, np.int64)
    args = (R, num_cols, nnz, rp, ci, vb, slices, block_rows, chunk_entries, hot_slots,
            hot_min_len, sizes)
    st = lib.orc_coo_blocked(*args, *([None] * 10))
    if st != OK:
        raise ValueError(f"orc_coo_blocked: status {st}")
    nch, ng, nw, nit, nbal = (int(v) for v in sizes)
    nblk = (R + block_rows - 1) // block_rows
    out = {"chunk_grp": np.zeros(nch + 1, np.int32), "chunk_blk": np.zeros(max(nch, 1), np.int32),
           "slice_chunk": np.zeros(slices + 1, np.int32),
           "slice_item": np.zeros(slices + 1, np.int32), "item_chunk": np.zeros(nit + 1, np.int32),
           "hot": np.zeros(max(nblk * hot_slots, 1), np.int32),
           "base": np.zeros(max(ng, 1), np.int32), "pk": np.zeros(max(64 * ng, 1), np.uint32),
           "val": np.zeros(max(64 * ng, 1), np.uint32), "wide": np.zeros(max(64 * nw, 1), np.int32)}
    st = lib.orc_coo_blocked(*args, *(out[k].ctypes.data for k in (
        "chunk_grp", "chunk_blk", "slice_chunk", "slice_item", "item_chunk", "hot", "base", "pk",
        "val", "wide")))
    assert st == OK
    out["chunk_blk"] = out["chunk_blk"][:nch]
    out["hot"] = out["hot"][:nblk * hot_slots]
    out["base"] = out["base"][:ng]
    out["pk"] = out["pk"][:64 * ng]
    out["val"] = out["val"][:64 * ng].view(np.float32)
    out["wide"] = out["wide"][:64 * nw]
    out["balanced_slices"] = nbal
    return out


def bc_block_rows(row_ptrs, col_idx, num_cols, slices, chunk_entries, hot_slots, hot_min_len):
    """Blocked COO block height for this matrix (orc_bc_block_rows)."""
    rp = _i32(row_ptrs)
    ci = _i32(col_idx)
    return int(_load().orc_bc_block_rows(rp.shape[0] - 1, num_cols, ci.shape[0], rp, ci,
                                         slices, chunk_entries, hot_slots, hot_min_len))


def bc_chunk_entries(nnz):
    """Blocked COO entries per chunk for a matrix of nnz nonzeros."""
    return int(_load().orc_bc_chunk_entries(int(nnz)))


def select_build(row_ptrs, col_idx, num_cols, block_rows):
    """The automatic build's (format name, K, lanes, x slices) for this matrix."""
    rp = _i32(row_ptrs)
    ci = _i32(col_idx)
    out = np.zeros(4, np.int64)
    st = _load().orc_select_build(rp.shape[0] - 1, num_cols, ci.shape[0], rp, ci, block_rows,
                                  out)
    assert st == OK
    return FMT_NAMES[int(out[0])], int(out[1]), int(out[2]), int(out[3])


def csr_to_sell(row_ptrs, col_idx, values, section=64):
    """Sectioned ELL (JDS variant): perm/len as JDS, section pointers, slots."""
    rp = _i32(row_ptrs)
    R = rp.shape[0] - 1
    lib = _load()
    slots = int(lib.orc_sell_slots(R, rp, section))
    if slots > 2**31 - 1:
        raise ValueError("too large")
    nsect = (R + section - 1) // section
    perm = np.empty(R, np.int32)
    slen = np.empty(R, np.int32)
    sptr = np.empty(nsect + 1, np.int32)
    sc = np.empty(slots, np.int32)
    sv = np.empty(slots, np.uint32)
    st = lib.orc_csr_to_sell(R, rp, _i32(col_idx), _bits(values), section, perm, slen, sptr,
                             sc, sv)
    if st == ERR_TOO_LARGE:
        raise ValueError("too large")
    return {"perm": perm, "len": slen, "sect_ptr": sptr, "col": sc, "val": sv.view(np.float32),
            "section": section}


# ------------------------------------------------------------------ selector

def hyb_width(num_rows, hist) -> int:
    h = np.ascontiguousarray(hist, np.int64)
    return int(_load().orc_hyb_width(num_rows, h.shape[0] - 1, h))


def vector_lanes(num_rows, nnz) -> int:
    return int(_load().orc_vector_lanes(num_rows, nnz))


def select(num_rows, nnz, hist, hyb_width_override: int = 0, lanes_override: int = 0):
    """Return (format name, K, lanes) chosen from the row-length statistics."""
    h = np.ascontiguousarray(hist, np.int64)
    out = np.zeros(3, np.int64)
    _load().orc_select(num_rows, nnz, h.shape[0] - 1, h, hyb_width_override, lanes_override, out)
    return FMT_NAMES[int(out[0])], int(out[1]), int(out[2])


# ------------------------------------------------------------------ CG

def cg(row_ptrs, col_idx, values, b, x0=None, max_iter=1000, rtol=1e-6):
    """Conjugate gradient for A x = b in fp64.  Returns (x, iterations, ||r||/||b||)."""
    rp = _i32(row_ptrs)
    R = rp.shape[0] - 1
    x = (np.zeros(R, np.float64) if x0 is None else np.array(x0, np.float64, copy=True))
    out = np.zeros(2, np.float64)
    _load().orc_cg(R, rp, _i32(col_idx), _f32(values), np.ascontiguousarray(b, np.float64), x,
                   int(max_iter), float(rtol), out)
    return x, int(out[0]), float(out[1])


# ------------------------------------------------------------------ OpenMP baseline

def _load_omp():
    global _omp
    if _omp is not None:
        return _omp
    build()
    lib = ctypes.CDLL(_OMP_LIB)
    lib.csr_omp_threads.restype = ctypes.c_int
    lib.csr_omp_threads.argtypes = []
    lib.csr_omp_bench.restype = ctypes.c_double
    lib.csr_omp_bench.argtypes = [_i64, _i64, _i32p, _i32p, _f32p, _f32p, _f32p, _f32p,
                                  ctypes.c_int, ctypes.c_int]
    _omp = lib
    return lib


def omp_threads() -> int:
    """Threads the OpenMP baseline runs with (OMP_NUM_THREADS or all cores)."""
    return int(_load_omp().csr_omp_threads())


def spmv_csr_omp(row_ptrs, col_idx, values, x, y, dynamic=False, reps=1):
    """OpenMP CSR baseline (fp32 row sums in row order, schedule static or
    dynamic,64): returns (fp32 y + A x, median seconds of `reps` timed runs)."""
    rp = _i32(row_ptrs)
    xs = _f32(x)
    out = np.empty(rp.shape[0] - 1, np.float32)
    t = _load_omp().csr_omp_bench(rp.shape[0] - 1, xs.shape[0], rp, _i32(col_idx),
                                  _f32(values), xs, _f32(y), out, 1 if dynamic else 0,
                                  int(reps))
    if t < 0:
        raise MemoryError("csr_omp_bench: allocation failed")
    return out, t
