"""Structure checks of the seeded synthetic workloads (CPU only)."""
import hashlib

import numpy as np
import pytest

from spmv_storage_formats_amd import synth


def _sha(w):
    h = hashlib.sha256()
    for a in (w.row_ptrs, w.col_idx, w.values, w.x, w.y):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def _rows_distinct_sorted(w):
    rows = np.repeat(np.arange(w.num_rows), np.diff(w.row_ptrs))
    key = rows.astype(np.int64) * w.num_cols + w.col_idx
    return bool(np.all(np.diff(key) > 0))


def _common(w):
    assert w.row_ptrs.dtype == np.int32 and w.col_idx.dtype == np.int32
    assert w.values.dtype == np.float32 and w.x.dtype == np.float32 and w.y.dtype == np.float32
    assert w.row_ptrs[0] == 0 and w.row_ptrs[-1] == w.nnz
    assert np.all(np.diff(w.row_ptrs) >= 0)
    assert w.col_idx.min() >= 0 and w.col_idx.max() < w.num_cols
    assert w.x.shape == (w.num_cols,) and w.y.shape == (w.num_rows,)
    assert np.all(np.abs(w.x) <= 1) and np.all(np.abs(w.y) <= 1)


def test_laplacian_full():
    w = synth.workload("c1")
    _common(w)
    assert (w.num_rows, w.nnz) == (65536, 326656)
    assert _rows_distinct_sorted(w)
    rows = np.repeat(np.arange(w.num_rows), np.diff(w.row_ptrs))
    diag = rows == w.col_idx
    assert np.all(w.values[diag] == 4) and np.all(w.values[~diag] == -1)
    assert diag.sum() == 65536


def test_random_rows_full():
    w = synth.workload("c2")
    _common(w)
    assert (w.num_rows, w.num_cols, w.nnz) == (1_000_000, 1_000_000, 5_000_000)
    assert np.array_equal(w.row_ptrs, 5 * np.arange(1_000_001, dtype=np.int32))
    assert _rows_distinct_sorted(w)
    assert np.all(np.abs(w.values) <= 1)


@pytest.mark.slow
def test_stencil27_full():
    w = synth.workload("c3")
    _common(w)
    assert (w.num_rows, w.nnz) == (2_097_152, 55_742_968)
    hist = np.bincount(np.diff(w.row_ptrs))
    assert {k: int(v) for k, v in enumerate(hist) if v} == {
        8: 8, 12: 1512, 18: 95256, 27: 2000376}
    assert _rows_distinct_sorted(w)


@pytest.mark.slow
def test_skewed_full():
    w = synth.workload("c4")
    _common(w)
    lens = np.diff(w.row_ptrs)
    long_rows = np.nonzero(lens > 20)[0]
    assert long_rows.tolist() == w.meta["long_rows"] and len(long_rows) == 50
    assert lens[long_rows].min() >= 1000 and lens[long_rows].max() <= 5000
    short = np.delete(lens, long_rows)
    assert short.min() == 10 and short.max() == 20
    assert _rows_distinct_sorted(w)


@pytest.mark.slow
def test_power_law_full():
    w = synth.workload("c5")
    _common(w)
    lens = np.diff(w.row_ptrs)
    assert w.num_rows == 4_000_000
    assert lens.min() == 2 and lens.max() < 100_000
    assert 15.0 < lens.mean() < 17.5
    assert 55e6 < w.nnz < 72e6
    assert np.all(w.values > 0) and np.all(w.values <= 1)
    assert _rows_distinct_sorted(w)


@pytest.mark.parametrize("name", ["c1s", "c2s", "c3s", "c4s", "c5s"])
def test_reduced_workloads(name):
    w = synth.workload(name)
    _common(w)
    assert _rows_distinct_sorted(w)


def test_deterministic():
    assert _sha(synth.workload("c2s")) == _sha(synth.workload("c2s"))
    assert _sha(synth.workload("c5s")) == _sha(synth.workload("c5s"))
    assert _sha(synth.workload("c4s")) != _sha(synth.skewed(200_001, 7, seed=99))


def test_power_law_mean_length():
    """The floored truncated Pareto(1.1) on [x_m, 100000) has mean 16."""
    a, xm, cap = 1.1, synth.POWER_LAW_XM, 1e5
    A, B = xm ** -a, cap ** -a
    k = np.arange(1, 100_000, dtype=np.float64)
    tail = np.where(k <= xm, 1.0, (k ** -a - B) / (A - B))  # P(len >= k)
    assert abs(tail.sum() - 16.0) < 1e-5


def test_max_band_structure():
    """Small instance of the int32-limit generator: nnz = R*per_row - 1, entry d
    of row r in column (r + d*R/per_row) mod R with value v[d]; the torch
    builder (run on the CPU here) gives the same arrays as the host rows."""
    torch = pytest.importorskip("torch")
    R, P = 64, 4
    m = synth.max_band(R, P, seed=6)
    w = m.to_workload()
    assert w.nnz == m.nnz == R * P - 1
    lens = w.lengths()
    assert np.all(lens[:-1] == P) and lens[-1] == P - 1
    for r in (0, 1, 17, R - 1):
        s, e = w.row_ptrs[r], w.row_ptrs[r + 1]
        d = np.arange(e - s)
        assert np.array_equal(w.col_idx[s:e], (r + d * (R // P)) % R)
        assert np.array_equal(w.values[s:e], m.v[d])
    rp, ci, v = m.csr_tensors(torch, "cpu")
    assert np.array_equal(rp.numpy(), w.row_ptrs)
    assert np.array_equal(ci.numpy(), w.col_idx)
    assert np.array_equal(v.numpy().view(np.uint32), w.values.view(np.uint32))


def test_max_band_default_size_is_int32_max():
    m = synth.max_band()
    assert m.nnz == np.iinfo(np.int32).max and m.x.shape == (2**26,)
