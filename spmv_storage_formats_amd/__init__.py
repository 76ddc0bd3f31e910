"""MI355X (gfx950) sparse matrix-vector multiply-accumulate engine, y <- A*x + y.

Thin Python binding over the C ABI of ``include/spmv.h``.  This module only
marshals arguments: every step (validation, statistics, format building, the
SpMV itself) runs in the HIP library ``libspmv_mi355x.so`` built from
``csrc/``.  There is no CPU fallback: if the library cannot be loaded, every
call raises.

    import torch, spmv_storage_formats_amd as spmv
    h = spmv.build("auto", row_ptrs, col_idx, values, num_cols)   # cuda tensors
    h.run(x, y)                  # y += A x on torch's current stream
"""
from __future__ import annotations

import ctypes
import os
import re
import sys
import threading

import numpy as np

__all__ = ["SpmvError", "Handle", "FORMATS", "ARRAYS", "load_library", "analyze", "select",
           "build", "build_coo", "build_tuned", "coo_to_csr", "library_path",
           "declared_functions"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
_LIB_PATH = os.path.join(_PKG, "libspmv_mi355x.so")
_HEADER = os.path.join(_ROOT, "include", "spmv.h")

FORMATS = {"auto": 0, "coo_atomic": 1, "coo_segmented": 2, "csr_scalar": 3, "csr_vector": 4,
           "ell": 5, "hyb": 6, "jds": 7, "csr_merge": 8, "sell": 9, "ell_xtile": 10,
           "coo_blocked": 11}
FORMAT_NAMES = {v: k for k, v in FORMATS.items()}
# name -> (enum value, numpy dtype)
ARRAYS = {
    "row_ptrs": (0, np.int32), "col_idx": (1, np.int32), "values": (2, np.float32),
    "row_idx": (3, np.int32), "ell_col": (4, np.int32), "ell_val": (5, np.float32),
    "ell_nnz": (6, np.int32), "tail_row": (7, np.int32), "tail_col": (8, np.int32),
    "tail_val": (9, np.float32), "jds_perm": (10, np.int32), "jds_len": (11, np.int32),
    "jds_iter_ptr": (12, np.int32), "jds_col": (13, np.int32), "jds_val": (14, np.float32),
    "len_hist": (15, np.int64), "sell_sect_ptr": (16, np.int32), "sell_col": (17, np.int32),
    "sell_val": (18, np.float32), "xt_run_ptr": (19, np.int32), "xt_runs": (20, np.int32),
    "xt_lidx": (21, np.int16), "bc_chunk_grp": (22, np.int32), "bc_chunk_blk": (23, np.int32),
    "bc_slice_chunk": (24, np.int32), "bc_hot": (25, np.int32), "bc_base": (26, np.int32),
    "bc_pk": (27, np.uint32), "bc_val": (28, np.float32), "bc_wide": (29, np.int32),
    "bc_slice_item": (30, np.int32), "bc_item_chunk": (31, np.int32),
}
CG_NOALLOC_MAX_ROWS = 1048576   # SPMV_CG_NOALLOC_MAX_ROWS in include/spmv.h
BC_BLOCK_ROWS = 32768           # SPMV_BC_BLOCK_ROWS: blocked COO rows per row block
BC_BLOCK_ROWS_TALL = 38912      # SPMV_BC_BLOCK_ROWS_TALL: blocks of balanced layouts
STATUS = {0: "SPMV_OK", 1: "SPMV_ERR_INVALID_ARG", 2: "SPMV_ERR_BAD_ROWPTRS",
          3: "SPMV_ERR_BAD_COLIDX", 4: "SPMV_ERR_BAD_ROWIDX", 5: "SPMV_ERR_TOO_LARGE",
          6: "SPMV_ERR_OOM", 7: "SPMV_ERR_HIP", 8: "SPMV_ERR_DEVICE"}


class SpmvError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = int(status)
        self.name = STATUS.get(self.status, f"status {status}")
        msg = _status_string(self.status)
        super().__init__(f"{what}: {self.name} ({msg})" if what else f"{self.name} ({msg})")


class _Opts(ctypes.Structure):
    _fields_ = [("hyb_width", ctypes.c_int32), ("lanes_per_row", ctypes.c_int32),
                ("validate", ctypes.c_int32), ("jds_depth", ctypes.c_int32),
                ("col_blocks", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("max_bytes", ctypes.c_int64)]


class _Stats(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int64), ("num_cols", ctypes.c_int64),
                ("nnz", ctypes.c_int64), ("max_len", ctypes.c_int64),
                ("sum_len_sq", ctypes.c_int64), ("empty_rows", ctypes.c_int64),
                ("col_spread", ctypes.c_int64)]


class _Info(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("hyb_width", ctypes.c_int32),
                ("lanes_per_row", ctypes.c_int32), ("ell_width", ctypes.c_int32),
                ("col_blocks", ctypes.c_int32), ("slice_cols", ctypes.c_int32),
                ("stats", _Stats), ("tail_nnz", ctypes.c_int64), ("num_tiles", ctypes.c_int64),
                ("device_bytes", ctypes.c_int64), ("groups", ctypes.c_int64),
                ("wide_groups", ctypes.c_int64), ("block_rows", ctypes.c_int32),
                ("chunk_entries", ctypes.c_int32), ("hot_slots", ctypes.c_int32),
                ("hot_min_len", ctypes.c_int32), ("work_items", ctypes.c_int32)]


class _TuneEntry(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("col_blocks", ctypes.c_int32),
                ("status", ctypes.c_int32), ("us", ctypes.c_float)]


TUNE_MAX = 32


class _TuneReport(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("chosen", ctypes.c_int32),
                ("entry", _TuneEntry * TUNE_MAX)]


_lock = threading.Lock()
_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


def library_path() -> str:
    return _LIB_PATH


def declared_functions() -> list[str]:
    """Names of the functions include/spmv.h declares (the library's exports)."""
    with open(_HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(spmv_[a-z_]+)\s*\(", text)))


def load_library():
    """Load the HIP library (building it in-tree first if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            from . import _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        sig = {
            "spmv_opts_default": (None, [P(_Opts)]),
            "spmv_analyze": (ctypes.c_int, [_i32, _i32, _i32, _vp, _vp, _i32, P(_Stats), _vp,
                                            ctypes.c_int64, _vp]),
            "spmv_select": (ctypes.c_int, [P(_Stats), _vp, P(_Opts), P(_i32), P(_i32), P(_i32)]),
            "spmv_build": (ctypes.c_int, [P(_vp), ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _vp,
                                          P(_Opts), _vp]),
            "spmv_build_coo": (ctypes.c_int, [P(_vp), ctypes.c_int, _i32, _i32, _i32, _vp, _vp,
                                              _vp, P(_Opts), _vp]),
            "spmv_coo_to_csr": (ctypes.c_int, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _i32, _vp]),
            "spmv_build_tuned": (ctypes.c_int, [P(_vp), _i32, _i32, _i32, _vp, _vp, _vp, P(_Opts),
                                                ctypes.c_uint32, _i32, P(_TuneReport), _vp]),
            "spmv_run": (ctypes.c_int, [_vp, _vp, _vp, _vp]),
            "spmv_cg": (ctypes.c_int, [_vp, _vp, _vp, _i32, ctypes.c_float, P(_i32),
                                       P(ctypes.c_float), _vp]),
            "spmv_cg_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _i32, ctypes.c_float, P(_i32),
                                               P(ctypes.c_float), _vp]),
            "spmv_get_info": (ctypes.c_int, [_vp, P(_Info)]),
            "spmv_array_bytes": (ctypes.c_int, [_vp, ctypes.c_int, P(ctypes.c_size_t)]),
            "spmv_export": (ctypes.c_int, [_vp, ctypes.c_int, _vp, ctypes.c_size_t]),
            "spmv_destroy": (ctypes.c_int, [_vp]),
            "spmv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "spmv_format_name": (ctypes.c_char_p, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _status_string(st: int) -> str:
    try:
        return load_library().spmv_status_string(st).decode()
    except Exception:  # pragma: no cover - library not loadable
        return "?"


def _check(st: int, what: str):
    if st != 0:
        raise SpmvError(st, what)


def _opts(hyb_width=0, lanes=0, validate=True, jds_depth=0, max_bytes=0, col_blocks=0) -> _Opts:
    return _Opts(int(hyb_width), int(lanes), 1 if validate else 0, int(jds_depth),
                 int(col_blocks), 0, int(max_bytes))


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}; one of {sorted(FORMATS)}")
        return FORMATS[fmt]
    return int(fmt)


def _dev(t, dtype, name, length=None):
    """Device pointer of a contiguous cuda tensor of `dtype` (0 if empty)."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a cuda tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if length is not None and t.numel() != length:
        raise ValueError(f"{name} has {t.numel()} elements, expected {length}")
    return t.data_ptr() if t.numel() else None


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _stats_dict(st: _Stats) -> dict:
    return {k: int(getattr(st, k)) for k, _ in _Stats._fields_}


def analyze(row_ptrs, col_idx, num_cols: int, validate: bool = True, stream=None) -> dict:
    """Input checks + row statistics on the device.  Returns the stats and
    the row-length histogram (numpy int64[max_len + 1])."""
    import torch
    lib = load_library()
    R = row_ptrs.numel() - 1
    rp = _dev(row_ptrs, torch.int32, "row_ptrs")
    ci = _dev(col_idx, torch.int32, "col_idx")
    st = _Stats()
    s = _stream(stream, row_ptrs.device)
    _check(lib.spmv_analyze(R, num_cols, col_idx.numel(), rp, ci, 1 if validate else 0,
                            ctypes.byref(st), None, 0, s), "spmv_analyze")
    hist = np.zeros(st.max_len + 1, np.int64)
    _check(lib.spmv_analyze(R, num_cols, col_idx.numel(), rp, ci, 0, ctypes.byref(st),
                            hist.ctypes.data, hist.size, s), "spmv_analyze")
    out = _stats_dict(st)
    out["hist"] = hist
    return out


def select(stats: dict, hist, hyb_width: int = 0, lanes: int = 0):
    """The library's format selector (host function): (format, K, lanes)."""
    lib = load_library()
    st = _Stats(*(int(stats[k]) for k, _ in _Stats._fields_))
    h = np.ascontiguousarray(hist, np.int64)
    if h.size != st.max_len + 1:
        raise ValueError("hist must have max_len + 1 entries")
    f, K, L = _i32(), _i32(), _i32()
    o = _opts(hyb_width, lanes)
    _check(lib.spmv_select(ctypes.byref(st), h.ctypes.data, ctypes.byref(o), ctypes.byref(f),
                           ctypes.byref(K), ctypes.byref(L)), "spmv_select")
    return FORMAT_NAMES[f.value], K.value, L.value


class Handle:
    """A built matrix.  Owns device copies of its format arrays."""

    def __init__(self, ptr: int, device):
        self._ptr = ctypes.c_void_p(ptr)
        self.device = device
        lib = load_library()
        info = _Info()
        _check(lib.spmv_get_info(self._ptr, ctypes.byref(info)), "spmv_get_info")
        self.info = {"format": FORMAT_NAMES[info.format], "hyb_width": info.hyb_width,
                     "lanes_per_row": info.lanes_per_row, "ell_width": info.ell_width,
                     "col_blocks": info.col_blocks, "slice_cols": info.slice_cols,
                     "tail_nnz": info.tail_nnz, "num_tiles": info.num_tiles,
                     "device_bytes": info.device_bytes, "groups": info.groups,
                     "wide_groups": info.wide_groups, "block_rows": info.block_rows,
                     "chunk_entries": info.chunk_entries, "hot_slots": info.hot_slots,
                     "hot_min_len": info.hot_min_len, "work_items": info.work_items,
                     **_stats_dict(info.stats)}

    @property
    def format(self) -> str:
        return self.info["format"]

    @property
    def num_rows(self) -> int:
        return self.info["num_rows"]

    @property
    def num_cols(self) -> int:
        return self.info["num_cols"]

    @property
    def nnz(self) -> int:
        return self.info["nnz"]

    def run(self, x, y, stream=None):
        """y <- A x + y, enqueued on `stream` (default: torch's current stream)."""
        import torch
        if self._ptr is None:
            raise RuntimeError("handle destroyed")
        xp = _dev(x, torch.float32, "x", self.num_cols)
        yp = _dev(y, torch.float32, "y", self.num_rows)
        if xp is not None and yp is not None:
            xs, xe = xp, xp + 4 * self.num_cols
            ys, ye = yp, yp + 4 * self.num_rows
            if xs < ye and ys < xe:
                raise ValueError("x and y must not overlap")
        _check(load_library().spmv_run(self._ptr, xp, yp, _stream(stream, y.device)),
               "spmv_run")
        return y

    def cg(self, b, x, max_iter: int = 1000, rtol: float = 1e-6, stream=None):
        """Conjugate gradient for A x = b (A square, symmetric positive definite).
        x holds the initial guess and receives the solution.  Returns
        (iterations, ||b - A x|| / ||b|| of the recurrence)."""
        import torch
        bp = _dev(b, torch.float32, "b", self.num_rows)
        xp = _dev(x, torch.float32, "x", self.num_rows)
        it = _i32()
        rr = ctypes.c_float()
        _check(load_library().spmv_cg(self._ptr, bp, xp, int(max_iter), float(rtol),
                                      ctypes.byref(it), ctypes.byref(rr),
                                      _stream(stream, x.device)), "spmv_cg")
        return it.value, rr.value

    def cg_noalloc(self, b, x, max_iter: int = 1000, rtol: float = 1e-6, stream=None):
        """The same solve as cg() on the library's static per-GPU workspace
        (spmv_cg_noalloc: no device allocation, at most CG_NOALLOC_MAX_ROWS rows;
        calls overlapping on one GPU race)."""
        import torch
        bp = _dev(b, torch.float32, "b", self.num_rows)
        xp = _dev(x, torch.float32, "x", self.num_rows)
        it = _i32()
        rr = ctypes.c_float()
        _check(load_library().spmv_cg_noalloc(self._ptr, bp, xp, int(max_iter), float(rtol),
                                              ctypes.byref(it), ctypes.byref(rr),
                                              _stream(stream, x.device)), "spmv_cg_noalloc")
        return it.value, rr.value

    def array(self, name: str) -> np.ndarray:
        """Copy one of the handle's arrays to a numpy array (bit-exact)."""
        which, dtype = ARRAYS[name]
        lib = load_library()
        n = ctypes.c_size_t()
        _check(lib.spmv_array_bytes(self._ptr, which, ctypes.byref(n)), "spmv_array_bytes")
        out = np.empty(n.value // np.dtype(dtype).itemsize, dtype)
        _check(lib.spmv_export(self._ptr, which, out.ctypes.data if out.size else None,
                               n.value), "spmv_export")
        return out

    def has_array(self, name: str) -> bool:
        n = ctypes.c_size_t()
        _check(load_library().spmv_array_bytes(self._ptr, ARRAYS[name][0], ctypes.byref(n)),
               "spmv_array_bytes")
        return n.value > 0 or name == "len_hist"

    def close(self):
        if sys.is_finalizing():
            return  # the HIP runtime may already be gone; the process frees it
        if getattr(self, "_ptr", None) is not None and _lib is not None:
            _lib.spmv_destroy(self._ptr)
        self._ptr = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def build(fmt, row_ptrs, col_idx, values, num_cols: int, *, hyb_width: int = 0, lanes: int = 0,
          validate: bool = True, jds_depth: int = 0, max_bytes: int = 0, col_blocks: int = 0,
          stream=None) -> Handle:
    """Build a handle in `fmt` ("auto" = selector) from CSR cuda tensors."""
    import torch
    lib = load_library()
    R = row_ptrs.numel() - 1
    nnz = col_idx.numel()
    rp = _dev(row_ptrs, torch.int32, "row_ptrs")
    ci = _dev(col_idx, torch.int32, "col_idx")
    va = _dev(values, torch.float32, "values", nnz)
    out = ctypes.c_void_p()
    o = _opts(hyb_width, lanes, validate, jds_depth, max_bytes, col_blocks)
    _check(lib.spmv_build(ctypes.byref(out), _fmt(fmt), R, int(num_cols), nnz, rp, ci, va,
                          ctypes.byref(o), _stream(stream, row_ptrs.device)), "spmv_build")
    return Handle(out.value, row_ptrs.device)


def build_coo(fmt, row_idx, col_idx, values, num_rows: int, num_cols: int, *, hyb_width: int = 0,
              lanes: int = 0, validate: bool = True, jds_depth: int = 0, max_bytes: int = 0,
              col_blocks: int = 0, stream=None) -> Handle:
    """Build a handle from COO cuda tensors (converted to CSR on the device)."""
    import torch
    lib = load_library()
    nnz = col_idx.numel()
    ri = _dev(row_idx, torch.int32, "row_idx", nnz)
    ci = _dev(col_idx, torch.int32, "col_idx")
    va = _dev(values, torch.float32, "values", nnz)
    out = ctypes.c_void_p()
    o = _opts(hyb_width, lanes, validate, jds_depth, max_bytes, col_blocks)
    _check(lib.spmv_build_coo(ctypes.byref(out), _fmt(fmt), int(num_rows), int(num_cols), nnz,
                              ri, ci, va, ctypes.byref(o), _stream(stream, col_idx.device)),
           "spmv_build_coo")
    return Handle(out.value, col_idx.device)


def coo_to_csr(row_idx, col_idx, values, num_rows: int, num_cols: int, validate: bool = True,
               stream=None):
    """COO -> CSR on the device.  Returns (row_ptrs, col_idx, values) tensors."""
    import torch
    lib = load_library()
    nnz = col_idx.numel()
    dev = col_idx.device
    rp = torch.empty(num_rows + 1, dtype=torch.int32, device=dev)
    co = torch.empty(nnz, dtype=torch.int32, device=dev)
    vo = torch.empty(nnz, dtype=torch.float32, device=dev)
    _check(lib.spmv_coo_to_csr(int(num_rows), int(num_cols), nnz,
                               _dev(row_idx, torch.int32, "row_idx", nnz),
                               _dev(col_idx, torch.int32, "col_idx"),
                               _dev(values, torch.float32, "values", nnz),
                               rp.data_ptr(), _dev(co, torch.int32, "out"),
                               _dev(vo, torch.float32, "out"), 1 if validate else 0,
                               _stream(stream, dev)), "spmv_coo_to_csr")
    return rp, co, vo


def build_tuned(row_ptrs, col_idx, values, num_cols: int, *, formats=None, runs: int = 5,
                hyb_width: int = 0, lanes: int = 0, validate: bool = True, jds_depth: int = 0,
                stream=None):
    """Empirical selector: time every candidate format on this matrix, keep the
    fastest.  Returns (handle, report) where report is a list of dicts
    {format, col_blocks, status, us} and report[i]["chosen"] marks the winner."""
    import torch
    lib = load_library()
    R = row_ptrs.numel() - 1
    nnz = col_idx.numel()
    mask = 0
    for f in (formats or []):
        mask |= 1 << _fmt(f)
    out = ctypes.c_void_p()
    rep = _TuneReport()
    o = _opts(hyb_width, lanes, validate, jds_depth, 0, 0)
    _check(lib.spmv_build_tuned(ctypes.byref(out), R, int(num_cols), nnz,
                                _dev(row_ptrs, torch.int32, "row_ptrs"),
                                _dev(col_idx, torch.int32, "col_idx"),
                                _dev(values, torch.float32, "values", nnz), ctypes.byref(o),
                                mask, int(runs), ctypes.byref(rep),
                                _stream(stream, row_ptrs.device)), "spmv_build_tuned")
    report = []
    for i in range(rep.count):
        e = rep.entry[i]
        report.append({"format": FORMAT_NAMES[e.format], "col_blocks": e.col_blocks,
                       "status": STATUS.get(e.status, e.status), "us": float(e.us),
                       "chosen": i == rep.chosen})
    return Handle(out.value, row_ptrs.device), report
