"""Seeded synthetic workloads for the SpMV engine and its checks.

Every matrix is produced directly in CSR form (row pointers, column indices,
fp32 values) together with dense fp32 vectors x and y.  This module only draws
random structure and values; it performs no SpMV and no format conversion, so
the GPU path and the CPU oracle can both consume its output without sharing any
of the method's arithmetic.

The shapes follow the workloads the source pages describe:

* ``laplacian2d``  -- the stencil solver that motivates SpMV inside iterative
  methods (PMPP notes, "Sparse Matrices and Basic Formats (COO & CSR)",
  background on SpMV and conjugate gradient).
* ``random_rows``  -- n x n matrix with a fixed small number of random columns
  per row, the illustrative 1M x 1M / 5M-nonzero case of the "Introduction to
  sparse computing" page, section on building the problem framework.
* ``stencil27``    -- FEM/CFD-like banded matrix with near-uniform rows, the
  regime where the SpMV format-choice article (section 3.1, 5.1) recommends ELL.
* ``skewed``       -- 99% of rows short, a few rows very long: the matrix of the
  SpMV format-choice article, section 4.1 (HYB with ELL width 20).
* ``power_law``    -- graph adjacency with Zipf row lengths: the social-network
  case of the SpMV format-choice article, sections 2.1 and 5.2.

Seeds: workload k uses ``SeedSequence(k).spawn(4)`` -> (structure, values, x, y).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "fig14_1",
    "laplacian2d",
    "random_rows",
    "stencil27",
    "skewed",
    "power_law",
    "small_random",
    "max_band",
    "BandMatrix",
    "workload",
    "WORKLOADS",
]


@dataclass
class Workload:
    name: str
    num_rows: int
    num_cols: int
    row_ptrs: np.ndarray  # int32 [R+1]
    col_idx: np.ndarray   # int32 [nnz]
    values: np.ndarray    # float32 [nnz]
    x: np.ndarray         # float32 [C]
    y: np.ndarray         # float32 [R]
    meta: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.col_idx.shape[0])

    def lengths(self) -> np.ndarray:
        """Row lengths, read back from the row pointers (input description only)."""
        return np.diff(self.row_ptrs.astype(np.int64))


def _streams(seed: int):
    ss = np.random.SeedSequence(seed).spawn(4)
    return [np.random.default_rng(s) for s in ss]


def _ptrs_from_lengths(lengths: np.ndarray) -> np.ndarray:
    out = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=out[1:])
    if out[-1] > np.iinfo(np.int32).max:
        raise ValueError("nnz exceeds int32")
    return out.astype(np.int32)


def _distinct_sorted_columns(rng, lengths: np.ndarray, num_cols: int) -> np.ndarray:
    """Per row, `lengths[r]` distinct columns uniform over [0, num_cols), ascending.

    Columns are drawn with replacement, duplicates inside a row are redrawn
    until none remain, then each row is sorted.  Sorting the composite key
    row*C + col keeps rows grouped and orders columns inside each row.
    """
    R = lengths.shape[0]
    if np.any(lengths > num_cols):
        raise ValueError("row longer than the number of columns")
    nnz = int(lengths.sum())
    row_base = np.repeat(np.arange(R, dtype=np.int64) * num_cols, lengths)
    cols = rng.integers(0, num_cols, size=nnz, dtype=np.int64)
    while True:
        key = np.sort(row_base + cols)
        cols = key - row_base
        dup = np.nonzero(key[1:] == key[:-1])[0] + 1
        if dup.size == 0:
            break
        cols[dup] = rng.integers(0, num_cols, size=dup.size, dtype=np.int64)
    return cols.astype(np.int32)


def _vec(rng, n: int) -> np.ndarray:
    return rng.uniform(-1.0, 1.0, size=n).astype(np.float32)


def fig14_1() -> Workload:
    """The 4x4 example matrix of Fig. 14.1 (PMPP notes, COO & CSR page).

    rows: [1 7 . .], [5 . 3 9], [. 2 8 .], [. . . 6].  The page prints no x or y;
    x = [1, 2, 3, 4] and y = 0 are chosen here (integers, so every result is exact).
    """
    row_ptrs = np.array([0, 2, 5, 7, 8], dtype=np.int32)
    col_idx = np.array([0, 1, 0, 2, 3, 1, 2, 3], dtype=np.int32)
    values = np.array([1, 7, 5, 3, 9, 2, 8, 6], dtype=np.float32)
    return Workload("fig14_1", 4, 4, row_ptrs, col_idx, values,
                    np.array([1, 2, 3, 4], dtype=np.float32),
                    np.zeros(4, dtype=np.float32), {"seed": None})


def laplacian2d(n: int = 256, seed: int = 1) -> Workload:
    """2-D 5-point Laplacian on an n x n grid, Dirichlet-truncated.

    Row r = i + n*j.  Entries in ascending column order: (i, j-1), (i-1, j),
    (i, j), (i+1, j), (i, j+1); diagonal 4, off-diagonals -1.
    """
    _, _, rx, ry = _streams(seed)
    R = n * n
    i = np.tile(np.arange(n), n)
    j = np.repeat(np.arange(n), n)
    r = np.arange(R, dtype=np.int64)
    cand_cols = np.stack([r - n, r - 1, r, r + 1, r + n], axis=1)
    cand_ok = np.stack([j > 0, i > 0, np.ones(R, bool), i < n - 1, j < n - 1], axis=1)
    cand_val = np.array([-1, -1, 4, -1, -1], dtype=np.float32)
    lengths = cand_ok.sum(axis=1)
    col_idx = cand_cols[cand_ok].astype(np.int32)
    values = np.broadcast_to(cand_val, (R, 5))[cand_ok].astype(np.float32)
    return Workload(f"laplacian2d_{n}", R, R, _ptrs_from_lengths(lengths), col_idx,
                    values, _vec(rx, R), _vec(ry, R), {"seed": seed, "grid": n})


def random_rows(num_rows: int = 1_000_000, per_row: int = 5, seed: int = 2) -> Workload:
    """Square matrix, exactly `per_row` distinct uniform random columns per row."""
    rs, rv, rx, ry = _streams(seed)
    lengths = np.full(num_rows, per_row, dtype=np.int64)
    col_idx = _distinct_sorted_columns(rs, lengths, num_rows)
    values = rv.uniform(-1.0, 1.0, size=col_idx.shape[0]).astype(np.float32)
    return Workload(f"random_rows_{num_rows}x{per_row}", num_rows, num_rows,
                    _ptrs_from_lengths(lengths), col_idx, values,
                    _vec(rx, num_rows), _vec(ry, num_rows),
                    {"seed": seed, "per_row": per_row})


def stencil27(n: int = 128, seed: int = 3) -> Workload:
    """3-D 27-point stencil on an n^3 grid, truncated at the faces.

    Row r = i + n*j + n*n*k; neighbour offsets (di, dj, dk) in {-1,0,1}^3 kept
    when inside the grid; columns ascending; values N(0, 1).
    """
    _, rv, rx, ry = _streams(seed)
    R = n ** 3
    r = np.arange(R, dtype=np.int64)
    i = r % n
    j = (r // n) % n
    k = r // (n * n)
    cols, oks = [], []
    for dk in (-1, 0, 1):
        for dj in (-1, 0, 1):
            for di in (-1, 0, 1):
                ok = ((i + di >= 0) & (i + di < n) & (j + dj >= 0) & (j + dj < n)
                      & (k + dk >= 0) & (k + dk < n))
                cols.append(r + di + n * dj + n * n * dk)
                oks.append(ok)
    cols = np.stack(cols, axis=1)
    oks = np.stack(oks, axis=1)
    lengths = oks.sum(axis=1)
    col_idx = cols[oks].astype(np.int32)
    del cols
    values = rv.standard_normal(size=col_idx.shape[0]).astype(np.float32)
    return Workload(f"stencil27_{n}", R, R, _ptrs_from_lengths(lengths), col_idx, values,
                    _vec(rx, R), _vec(ry, R), {"seed": seed, "grid": n})


def skewed(num_rows: int = 2_000_000, n_long: int = 50, short=(10, 20),
           long=(1000, 5000), seed: int = 4) -> Workload:
    """All rows U{short} long except `n_long` random rows of U{long} nonzeros."""
    rs, rv, rx, ry = _streams(seed)
    lengths = rs.integers(short[0], short[1] + 1, size=num_rows, dtype=np.int64)
    long_rows = rs.choice(num_rows, size=n_long, replace=False)
    lengths[long_rows] = rs.integers(long[0], long[1] + 1, size=n_long, dtype=np.int64)
    lengths = np.minimum(lengths, num_rows)
    col_idx = _distinct_sorted_columns(rs, lengths, num_rows)
    values = rv.uniform(-1.0, 1.0, size=col_idx.shape[0]).astype(np.float32)
    return Workload(f"skewed_{num_rows}", num_rows, num_rows, _ptrs_from_lengths(lengths),
                    col_idx, values, _vec(rx, num_rows), _vec(ry, num_rows),
                    {"seed": seed, "long_rows": np.sort(long_rows).tolist()})


# x_m of the truncated continuous Pareto(alpha = 1.1) whose floor has mean 16
# with cap 100000 (solved numerically; pmf of the floored lengths ~ k^-2.1).
POWER_LAW_XM = 2.2855465


def power_law(num_rows: int = 4_000_000, seed: int = 5, cap: int = 100_000,
              alpha: float = 1.1, x_m: float = POWER_LAW_XM) -> Workload:
    """Graph adjacency with Zipf(2.1)-like row lengths (min 2, below `cap`).

    len = floor(F^-1(U)) for the Pareto(alpha) law truncated to [x_m, cap):
    len = floor((A - U (A - B))^(-1/alpha)), A = x_m^-alpha, B = cap^-alpha.
    Rows come in i.i.d. order; values U(0, 1].
    """
    rs, rv, rx, ry = _streams(seed)
    A = x_m ** (-alpha)
    B = float(cap) ** (-alpha)
    u = rs.random(num_rows)
    lengths = np.floor((A - u * (A - B)) ** (-1.0 / alpha)).astype(np.int64)
    lengths = np.clip(lengths, 1, min(cap, num_rows))
    col_idx = _distinct_sorted_columns(rs, lengths, num_rows)
    values = (1.0 - rv.random(size=col_idx.shape[0])).astype(np.float32)
    return Workload(f"power_law_{num_rows}", num_rows, num_rows, _ptrs_from_lengths(lengths),
                    col_idx, values, _vec(rx, num_rows), _vec(ry, num_rows),
                    {"seed": seed, "cap": cap})


@dataclass
class BandMatrix:
    """The largest matrix int32 indices allow: ``num_rows`` rows of ``per_row``
    entries, the last row one shorter, so nnz = 2^31 - 1 at the defaults
    (2^26 rows of 32).

    Entry d of row r sits in column (r + d * (num_rows // per_row)) mod num_rows
    (a wrapped band: each row touches columns spread over the whole of x, in
    increasing order except where the band wraps) and has value v[d], one of
    ``per_row`` seeded U[-1, 1] values.  At full size the arrays (17 GB) are
    generated where they are used -- ``csr_tensors`` builds them with torch on
    the target device -- and ``row`` gives any row's entries on the host.
    """
    num_rows: int
    per_row: int
    v: np.ndarray   # float32 [per_row]
    x: np.ndarray   # float32 [num_rows]
    y: np.ndarray   # float32 [num_rows]

    @property
    def nnz(self) -> int:
        return self.num_rows * self.per_row - 1

    @property
    def stride(self) -> int:
        return self.num_rows // self.per_row

    def row(self, r: int):
        """(columns, values) of row r, in storage order."""
        n = self.per_row - (1 if r == self.num_rows - 1 else 0)
        d = np.arange(n, dtype=np.int64)
        cols = ((r + d * self.stride) % self.num_rows).astype(np.int32)
        return cols, self.v[:n].copy()

    def csr_tensors(self, torch, device):
        """(row_ptrs int32 [R+1], col_idx int32 [nnz], values fp32 [nnz]) on `device`."""
        R, P = self.num_rows, self.per_row
        rp = torch.arange(R + 1, dtype=torch.int64, device=device) * P
        rp[-1] -= 1
        base = torch.arange(R, dtype=torch.int32, device=device)
        offs = torch.arange(P, dtype=torch.int32, device=device) * self.stride
        cols = base[:, None] + offs[None, :]            # < 2R, no int32 overflow
        cols = torch.where(cols >= R, cols - R, cols)
        vals = torch.from_numpy(self.v).to(device)[None, :].expand(R, P).contiguous()
        return (rp.to(torch.int32), cols.reshape(-1)[:self.nnz],
                vals.reshape(-1)[:self.nnz])

    def to_workload(self) -> Workload:
        """Host CSR arrays (for small instances)."""
        lengths = np.full(self.num_rows, self.per_row, dtype=np.int64)
        lengths[-1] -= 1
        cols = np.concatenate([self.row(r)[0] for r in range(self.num_rows)])
        vals = np.concatenate([self.row(r)[1] for r in range(self.num_rows)])
        return Workload(f"max_band_{self.num_rows}x{self.per_row}", self.num_rows,
                        self.num_rows, _ptrs_from_lengths(lengths), cols, vals, self.x,
                        self.y, {"per_row": self.per_row})


def max_band(num_rows: int = 2**26, per_row: int = 32, seed: int = 6) -> BandMatrix:
    _, rv, rx, ry = _streams(seed)
    v = rv.uniform(-1.0, 1.0, size=per_row).astype(np.float32)
    return BandMatrix(num_rows, per_row, v, _vec(rx, num_rows), _vec(ry, num_rows))


def small_random(rng: np.random.Generator, num_rows: int, num_cols: int, max_len: int,
                 empty_frac: float = 0.2, duplicates: bool = True,
                 unsorted: bool = True, integer_values: bool = False) -> Workload:
    """Tiny irregular CSR for edge-case checks.

    Rows may be empty, may repeat a column (duplicates are kept as separate
    entries) and may list columns in any order.
    """
    lengths = rng.integers(0, max_len + 1, size=num_rows)
    lengths[rng.random(num_rows) < empty_frac] = 0
    if num_cols == 0:
        lengths[:] = 0
    nnz = int(lengths.sum())
    if num_cols > 0:
        if duplicates:
            cols = rng.integers(0, num_cols, size=nnz)
        else:
            lengths = np.minimum(lengths, num_cols)
            nnz = int(lengths.sum())
            cols = np.concatenate([rng.permutation(num_cols)[:l] for l in lengths]) \
                if nnz else np.zeros(0, np.int64)
        if not unsorted:
            rp = np.concatenate([[0], np.cumsum(lengths)])
            cols = np.concatenate([np.sort(cols[rp[r]:rp[r + 1]]) for r in range(num_rows)]) \
                if nnz else cols
    else:
        cols = np.zeros(0, np.int64)
    if integer_values:
        vals = rng.integers(-8, 9, size=nnz).astype(np.float32)
        x = rng.integers(-8, 9, size=num_cols).astype(np.float32)
        y = rng.integers(-8, 9, size=num_rows).astype(np.float32)
    else:
        vals = rng.uniform(-1, 1, size=nnz).astype(np.float32)
        x = rng.uniform(-1, 1, size=num_cols).astype(np.float32)
        y = rng.uniform(-1, 1, size=num_rows).astype(np.float32)
    return Workload(f"small_{num_rows}x{num_cols}", num_rows, num_cols,
                    _ptrs_from_lengths(lengths.astype(np.int64)),
                    np.asarray(cols, dtype=np.int32), vals, x, y, {})


# Full-size workloads (the five configurations) and reduced sizes that keep the
# same structure but finish in seconds on the CPU oracle.
WORKLOADS = {
    "c1": (lambda: laplacian2d(256, seed=1)),
    "c2": (lambda: random_rows(1_000_000, 5, seed=2)),
    "c3": (lambda: stencil27(128, seed=3)),
    "c4": (lambda: skewed(2_000_000, 50, seed=4)),
    "c5": (lambda: power_law(4_000_000, seed=5)),
    # reduced versions (several tiles and a ragged tail, seconds on the CPU)
    "c1s": (lambda: laplacian2d(61, seed=11)),
    "c2s": (lambda: random_rows(100_003, 5, seed=12)),
    "c3s": (lambda: stencil27(37, seed=13)),
    "c4s": (lambda: skewed(200_001, 7, seed=14)),
    "c5s": (lambda: power_law(300_007, seed=15, cap=30_000)),
}


def workload(name: str) -> Workload:
    if name == "fig14_1":
        return fig14_1()
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    return WORKLOADS[name]()
