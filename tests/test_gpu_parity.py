"""GPU parity: every builder and kernel of the HIP library against the CPU oracle.

Index arrays and moved values must match the oracle bit for bit; y must meet
the row bound |y_gpu - y_ref| <= 1e-5 * (|y| + sum |a*x|) on every row.
All calls go through the C ABI (the ctypes binding in spmv_storage_formats_amd).
"""
import numpy as np
import pytest

import oracle
from spmv_storage_formats_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import spmv_storage_formats_amd as spmv  # noqa: E402

ALL_FORMATS = ["coo_atomic", "coo_segmented", "csr_scalar", "csr_vector", "ell", "hyb", "jds",
               "csr_merge", "sell", "ell_xtile", "coo_blocked"]
# formats whose rows are each summed by one lane group with a plain y update
DETERMINISTIC = ["csr_scalar", "csr_vector", "ell", "ell_xtile"]

_cache = {}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spmv.load_library()
    return torch.device("cuda:0")


def xtile_refused(row_ptrs, col_idx, values):
    """Whether the oracle refuses the x-tile format for this CSR matrix."""
    try:
        oracle.csr_to_ell_xtile(row_ptrs, col_idx, values)
        return False
    except ValueError:
        return True


def expect_refused(fmt, w, dev, **kw):
    """For a format the oracle refuses on w: the build fails with TOO_LARGE."""
    with pytest.raises(spmv.SpmvError) as ei:
        build(fmt, w, dev, **kw)
    assert ei.value.name == "SPMV_ERR_TOO_LARGE"


def W(name):
    if name not in _cache:
        _cache[name] = synth.workload(name)
    return _cache[name]


def ref(name):
    key = ("ref", name)
    if key not in _cache:
        w = W(name)
        _cache[key] = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    return _cache[key]


def to_dev(w, dev):
    return (torch.from_numpy(w.row_ptrs).to(dev), torch.from_numpy(w.col_idx).to(dev),
            torch.from_numpy(w.values).to(dev), torch.from_numpy(w.x).to(dev),
            torch.from_numpy(w.y).to(dev))


def run_once(h, x, y0):
    y = y0.clone()
    h.run(x, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_rows(y_gpu, y_ref, bound, what):
    n, first, worst = oracle.check(y_gpu, y_ref, bound)
    assert n == 0, (f"{what}: {n} rows out of bound, first row {first}: gpu {y_gpu[first]!r} "
                    f"ref {y_ref[first]!r} bound {bound[first]!r}")
    return worst


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def build(fmt, w, dev, **kw):
    rp, ci, v, _, _ = to_dev(w, dev)
    return spmv.build(fmt, rp, ci, v, w.num_cols, **kw)


# --------------------------------------------------------------- worked example

@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_fig14_1_every_format(dev, fmt):
    w = synth.fig14_1()
    rp, ci, v, x, _ = to_dev(w, dev)
    h = spmv.build(fmt, rp, ci, v, 4)
    y = torch.zeros(4, device=dev)
    h.run(x, y)
    assert y.cpu().tolist() == [15, 50, 28, 24]
    y = torch.ones(4, device=dev)
    h.run(x, y)
    assert y.cpu().tolist() == [16, 51, 29, 25]


def test_fig14_1_sectioned_ell(dev):
    """Sections of 64 rows on Fig. 14.1: one section of the 4 sorted rows,
    width 3, pointers [0, 12]; the arrays equal the oracle's."""
    w = synth.fig14_1()
    h = build("sell", w, dev)
    assert h.array("sell_sect_ptr").tolist() == [0, 12]
    assert h.array("jds_perm").tolist() == [1, 0, 2, 3]
    check_builder(h, w)


def test_fig14_1_printed_arrays(dev):
    """Device builders reproduce the printed ELL and JDS arrays of Fig. 14.1."""
    w = synth.fig14_1()
    h = build("ell", w, dev)
    assert h.info["ell_width"] == 3
    assert h.array("ell_val").tolist() == [1, 5, 2, 6, 7, 3, 8, 0, 0, 9, 0, 0]
    assert h.array("ell_col").tolist() == [0, 0, 1, 3, 1, 2, 2, 0, 0, 3, 0, 0]
    assert h.array("ell_nnz").tolist() == [2, 3, 2, 1]
    h = build("jds", w, dev)
    assert h.array("jds_perm").tolist() == [1, 0, 2, 3]
    assert h.array("jds_iter_ptr").tolist() == [0, 4, 7, 8]
    assert h.array("jds_val").tolist() == [5, 1, 2, 6, 3, 7, 8, 9]
    h = build("hyb", w, dev, hyb_width=2)
    assert h.array("tail_row").tolist() == [1] and h.array("tail_val").tolist() == [9]
    assert build("auto", w, dev).format == "ell"


# -------------------------------------------------------------- builder parity

def check_builder(h, w, K=None):
    fmt = h.format
    if fmt in ("csr_scalar", "csr_vector", "csr_merge"):
        assert np.array_equal(h.array("row_ptrs"), w.row_ptrs)
        assert np.array_equal(h.array("col_idx"), w.col_idx)
        assert np.array_equal(bits(h.array("values")), bits(w.values))
    elif fmt in ("coo_atomic", "coo_segmented"):
        assert np.array_equal(h.array("row_idx"), oracle.csr_to_coo(w.row_ptrs))
        assert np.array_equal(h.array("col_idx"), w.col_idx)
        assert np.array_equal(bits(h.array("values")), bits(w.values))
    elif fmt == "ell":
        e = oracle.csr_to_ell(w.row_ptrs, w.col_idx, w.values)
        assert h.info["ell_width"] == e["width"]
        assert np.array_equal(h.array("ell_col"), e["col"])
        assert np.array_equal(bits(h.array("ell_val")), bits(e["val"]))
        assert np.array_equal(h.array("ell_nnz"), e["nnz"])
    elif fmt == "hyb":
        o = oracle.csr_to_hyb(w.row_ptrs, w.col_idx, w.values, h.info["hyb_width"])
        assert h.info["ell_width"] == o["width"]
        assert np.array_equal(h.array("ell_col"), o["ell_col"])
        assert np.array_equal(bits(h.array("ell_val")), bits(o["ell_val"]))
        assert np.array_equal(h.array("ell_nnz"), o["ell_nnz"])
        assert h.info["tail_nnz"] == o["tail_row"].size
        assert np.array_equal(h.array("tail_row"), o["tail_row"])
        assert np.array_equal(h.array("tail_col"), o["tail_col"])
        assert np.array_equal(bits(h.array("tail_val")), bits(o["tail_val"]))
    elif fmt == "jds":
        o = oracle.csr_to_jds(w.row_ptrs, w.col_idx, w.values)
        assert np.array_equal(h.array("jds_perm"), o["perm"])
        assert np.array_equal(h.array("jds_len"), o["len"])
        assert np.array_equal(h.array("jds_iter_ptr"), o["iter_ptr"])
        assert np.array_equal(h.array("jds_col"), o["col"])
        assert np.array_equal(bits(h.array("jds_val")), bits(o["val"]))
    elif fmt == "ell_xtile":
        o = oracle.csr_to_ell_xtile(w.row_ptrs, w.col_idx, w.values)
        assert h.info["ell_width"] == o["width"]
        assert np.array_equal(h.array("xt_run_ptr"), o["run_ptr"])
        assert np.array_equal(h.array("xt_runs"), o["runs"].reshape(-1))
        assert np.array_equal(h.array("xt_lidx"), o["lidx"])
        assert np.array_equal(bits(h.array("ell_val")), bits(o["val"]))
        assert np.array_equal(h.array("ell_nnz"), o["nnz"])
    elif fmt == "coo_blocked":
        check_blocked(h, w)
    elif fmt == "sell":
        o = oracle.csr_to_sell(w.row_ptrs, w.col_idx, w.values, 64)
        assert np.array_equal(h.array("jds_perm"), o["perm"])
        assert np.array_equal(h.array("jds_len"), o["len"])
        assert np.array_equal(h.array("sell_sect_ptr"), o["sect_ptr"])
        assert np.array_equal(h.array("sell_col"), o["col"])
        assert np.array_equal(bits(h.array("sell_val")), bits(o["val"]))
    st = oracle.row_stats(w.row_ptrs)
    assert np.array_equal(h.array("len_hist"), st["hist"])
    assert (h.info["max_len"], h.info["sum_len_sq"], h.info["empty_rows"]) == \
        (st["W"], st["sum_len_sq"], st["empty_rows"])


def check_blocked(h, w):
    """Every blocked-COO array equals the oracle's, built with the handle's own
    slice count, block height, chunk size and hot-row rule (spmv_info)."""
    i = h.info
    assert i["block_rows"] == oracle.bc_block_rows(w.row_ptrs, w.col_idx, w.num_cols,
                                                   i["col_blocks"], i["chunk_entries"],
                                                   i["hot_slots"], i["hot_min_len"])
    o = oracle.csr_to_coo_blocked(w.row_ptrs, w.col_idx, w.values, w.num_cols, i["col_blocks"],
                                  i["block_rows"], i["chunk_entries"], i["hot_slots"],
                                  i["hot_min_len"])
    assert i["slice_cols"] == max(-(-w.num_cols // i["col_blocks"]), 1)
    assert i["chunk_entries"] == oracle.bc_chunk_entries(w.nnz)
    assert i["num_tiles"] == o["chunk_blk"].size and i["groups"] == o["base"].size
    assert i["wide_groups"] * 64 == o["wide"].size
    assert i["work_items"] + 1 == o["item_chunk"].size
    for name in ("chunk_grp", "chunk_blk", "slice_chunk", "slice_item", "item_chunk", "hot",
                 "base", "pk", "wide"):
        assert np.array_equal(h.array("bc_" + name), o[name]), name
    assert np.array_equal(bits(h.array("bc_val")), bits(o["val"]))


REDUCED = ["c1s", "c2s", "c3s", "c4s", "c5s"]


@pytest.mark.parametrize("name", REDUCED)
@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_reduced_builders_and_spmv(dev, name, fmt):
    w = W(name)
    slots = w.num_rows * oracle.row_stats(w.row_ptrs)["W"]
    print(f"[case] {name} {fmt} R={w.num_rows} nnz={w.nnz}", flush=True)
    if fmt == "ell" and slots > 2**31 - 1:
        with pytest.raises(spmv.SpmvError) as ei:
            build(fmt, w, dev)
        assert ei.value.name == "SPMV_ERR_TOO_LARGE"
        return
    if fmt == "ell" and slots > 64_000_000:
        pytest.skip("ELL of this skewed shape is >99% padding (multi-GB); covered at full size")
    if fmt == "ell_xtile" and xtile_refused(w.row_ptrs, w.col_idx, w.values):
        expect_refused(fmt, w, dev)
        return
    h = build(fmt, w, dev)
    assert h.format == fmt
    check_builder(h, w)
    _, _, _, x, y0 = to_dev(w, dev)
    y_ref, bound = ref(name)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"{name}/{fmt}")


@pytest.mark.parametrize("K", [0, 1, 2, 5, 13, 20, 64, 100000])
def test_hyb_widths(dev, K):
    w = W("c4s")
    h = build("hyb", w, dev, hyb_width=K)
    check_builder(h, w)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), *ref("c4s"), f"hyb K={K}")


@pytest.mark.parametrize("lanes", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("name", ["c2s", "c4s", "c5s"])
def test_csr_vector_lanes(dev, lanes, name):
    w = W(name)
    h = build("csr_vector", w, dev, lanes=lanes)
    assert h.info["lanes_per_row"] == lanes
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), *ref(name), f"{name} lanes={lanes}")


@pytest.mark.parametrize("fmt", ["jds", "sell"])
@pytest.mark.parametrize("depth", [1, 3, 64, 128, 1000])
def test_jds_depths(dev, depth, fmt):
    w = W("c5s")
    h = build(fmt, w, dev, jds_depth=depth)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), *ref("c5s"), f"jds depth={depth}")


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_small_irregular(dev, seed, fmt):
    """Tiny matrices with empty rows, duplicate and unsorted columns, R != C."""
    rng = np.random.default_rng(100 + seed)
    R, C = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    w = synth.small_random(rng, R, C, max_len=int(rng.integers(1, 40)))
    h = build(fmt, w, dev)
    check_builder(h, w)
    y_ref, bound = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"small seed={seed} {fmt}")


# ----------------------------------------------------------------- edge cases

@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_empty_matrices(dev, fmt):
    for R, C in ((0, 0), (0, 5), (7, 3)):
        rp = torch.zeros(R + 1, dtype=torch.int32, device=dev)
        e = torch.zeros(0, dtype=torch.int32, device=dev)
        h = spmv.build(fmt, rp, e, torch.zeros(0, device=dev), C)
        y = torch.arange(R, dtype=torch.float32, device=dev)
        h.run(torch.ones(C, device=dev), y)
        assert y.cpu().tolist() == list(range(R))


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_one_huge_row(dev, fmt):
    """One 200k-long row among empty and short rows: the merge path spans
    ~100 blocks, JDS splits the row over many tiles."""
    rng = np.random.default_rng(5)
    R, C = 20000, 300_000          # R * 200000 > 2^31: ELL must be refused
    lens = rng.integers(0, 4, size=R)
    lens[1234] = 200_000
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ci = np.concatenate([np.sort(rng.choice(C, l, replace=False)) if l else np.zeros(0, np.int64)
                         for l in lens]).astype(np.int32)
    w = synth.Workload("huge_row", R, C, rp, ci, rng.uniform(-1, 1, ci.size).astype(np.float32),
                       rng.uniform(-1, 1, C).astype(np.float32),
                       rng.uniform(-1, 1, R).astype(np.float32))
    if fmt in ("ell", "ell_xtile") and R * 200_000 > 2**31 - 1:
        expect_refused(fmt, w, dev)
        return
    h = build(fmt, w, dev)
    check_builder(h, w)
    y_ref, bound = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"huge row {fmt}")


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_closed_forms(dev, fmt):
    """5-point Laplacian, x = 1, y = 0: 0 inside, 1 on edges, 2 at corners --
    exact in fp32 in any summation order; x = 0 leaves y bit-identical."""
    w = W("c1s")
    n = 61
    h = build(fmt, w, dev)
    y = torch.zeros(n * n, device=dev)
    h.run(torch.ones(n * n, device=dev), y)
    g = y.cpu().numpy().reshape(n, n)
    expect = np.zeros((n, n), np.float32)
    expect[0] += 1; expect[-1] += 1; expect[:, 0] += 1; expect[:, -1] += 1
    assert np.array_equal(g, expect)
    y0 = torch.from_numpy(w.y).to(dev)
    y = y0.clone()
    h.run(torch.zeros(n * n, device=dev), y)
    assert np.array_equal(bits(y.cpu().numpy()), bits(w.y))


@pytest.mark.parametrize("fmt", DETERMINISTIC)
def test_repeat_runs_bit_identical(dev, fmt):
    """Kernels without atomics give the same bits on every run (no races)."""
    w = W("c3s")
    h = build(fmt, w, dev)
    _, _, _, x, y0 = to_dev(w, dev)
    a = run_once(h, x, y0)
    for _ in range(3):
        assert np.array_equal(bits(run_once(h, x, y0)), bits(a))


def test_non_default_stream(dev):
    w = W("c2s")
    h = build("ell", w, dev)
    _, _, _, x, y0 = to_dev(w, dev)
    s = torch.cuda.Stream()
    y = y0.clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        h.run(x, y)
    s.synchronize()
    assert_rows(y.cpu().numpy(), *ref("c2s"), "side stream")


# ----------------------------------------------------------- analyze / validate

@pytest.mark.parametrize("name", ["fig14_1", "c1s", "c4s", "c5s"])
def test_analyze_matches_oracle(dev, name):
    w = synth.fig14_1() if name == "fig14_1" else W(name)
    rp, ci, _, _, _ = to_dev(w, dev)
    got = spmv.analyze(rp, ci, w.num_cols)
    st = oracle.row_stats(w.row_ptrs)
    assert (got["max_len"], got["nnz"], got["sum_len_sq"], got["empty_rows"]) == \
        (st["W"], st["nnz"], st["sum_len_sq"], st["empty_rows"])
    assert np.array_equal(got["hist"], st["hist"])


def _bad_inputs():
    w = synth.fig14_1()
    rp, ci = w.row_ptrs, w.col_idx
    cases = []
    b = rp.copy(); b[2] = 1; cases.append(("decreasing", b, ci, 4))
    b = rp.copy(); b[0] = 1; cases.append(("start", b, ci, 4))
    b = rp.copy(); b[4] = 9; cases.append(("end beyond nnz", b, ci.copy(), 4))
    cases.append(("nnz mismatch", rp.copy(), ci[:7].copy(), 4))
    b = ci.copy(); b[3] = 4; cases.append(("col high", rp.copy(), b, 4))
    b = ci.copy(); b[0] = -1; cases.append(("col negative", rp.copy(), b, 4))
    cases.append(("too few columns", rp.copy(), ci.copy(), 3))
    # pointers whose difference wraps in int32: INT32_MAX then INT32_MIN
    b = rp.copy(); b[1] = np.iinfo(np.int32).max; b[2] = np.iinfo(np.int32).min
    cases.append(("wrapping pair", b, ci.copy(), 4))
    # non-decreasing until a pointer far past nnz, then back down to nnz
    b = rp.copy(); b[2] = np.iinfo(np.int32).max; b[3] = np.iinfo(np.int32).max
    cases.append(("pointer past nnz", b, ci.copy(), 4))
    return cases


@pytest.mark.parametrize("case", range(9))
def test_validation_codes_match_oracle(dev, case):
    name, rp, ci, C = _bad_inputs()[case]
    expect = oracle.validate_csr(4, C, rp, ci)
    assert expect != oracle.OK
    vals = torch.ones(ci.size, device=dev)
    with pytest.raises(spmv.SpmvError) as ei:
        spmv.build("auto", torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev), vals, C)
    assert ei.value.status == expect, name


def test_validate_off_skips_column_pass(dev):
    w = synth.fig14_1()
    ci = w.col_idx.copy()
    ci[3] = 9  # out of range, not checked when validate=False (caller's promise)
    a = spmv.analyze(torch.from_numpy(w.row_ptrs).to(dev), torch.from_numpy(ci).to(dev), 4,
                     validate=False)
    assert a["max_len"] == 3


def test_too_large_and_budget(dev):
    w = W("c4s")
    R, Wd = w.num_rows, oracle.row_stats(w.row_ptrs)["W"]
    assert R * Wd < 2**31  # reduced skewed fits; the budget refuses it
    with pytest.raises(spmv.SpmvError) as ei:
        build("ell", w, dev, max_bytes=1 << 20)
    assert ei.value.name == "SPMV_ERR_TOO_LARGE"
    h = build("hyb", w, dev, max_bytes=1 << 30)
    assert h.info["device_bytes"] <= 1 << 30


def _one_long_row():
    """200 rows: row 0 holds 5,000 entries, the others one each."""
    rng = np.random.default_rng(5)
    lens = np.ones(200, np.int64)
    lens[0] = 5000
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ci = np.concatenate([np.sort(rng.choice(8000, l, replace=False)) for l in lens]).astype(np.int32)
    return rp, ci, rng.standard_normal(ci.size).astype(np.float32), 8000


@pytest.mark.parametrize("case", ALL_FORMATS + ["sliced", "coo_blocked_wide", "jds_depth1"])
def test_budget_bounds_the_built_arrays(dev, case):
    """opts.max_bytes bounds the device arrays a handle keeps: with a budget one
    byte below what the same build keeps, the build is refused with
    SPMV_ERR_TOO_LARGE; a build that succeeds under a budget keeps no more than
    it.  The wide-group blocked build and JDS at depth 1 are the cases whose
    size the pre-build estimate cannot see (wide groups; tiles per jagged
    column)."""
    kw = {}
    fmt = case
    if case == "coo_blocked_wide":
        w = _wide_mix()
        rp, ci, v, C = w.row_ptrs, w.col_idx, w.values, w.num_cols
        fmt = "coo_blocked"
    elif case == "jds_depth1":
        rp, ci, v, C = _one_long_row()
        fmt, kw = "jds", {"jds_depth": 1}
    else:
        w = W("c3s" if case == "ell_xtile" else "c2s")
        rp, ci, v, C = w.row_ptrs, w.col_idx, w.values, w.num_cols
        if case == "sliced":
            fmt, kw = "csr_merge", {"col_blocks": 3}
    t = [torch.from_numpy(a).to(dev) for a in (rp, ci, v)]
    h = spmv.build(fmt, *t, C, **kw)
    need = h.info["device_bytes"]
    if case == "coo_blocked_wide":
        assert h.info["wide_groups"] > 0
    h.close()
    with pytest.raises(spmv.SpmvError) as ei:
        spmv.build(fmt, *t, C, max_bytes=need - 1, **kw)
    assert ei.value.name == "SPMV_ERR_TOO_LARGE"
    try:
        h = spmv.build(fmt, *t, C, max_bytes=need, **kw)
    except spmv.SpmvError as e:   # the pre-build estimate may be an overestimate
        assert e.name == "SPMV_ERR_TOO_LARGE"
    else:
        assert h.info["device_bytes"] <= need
        h.close()


# ------------------------------------------------------------------ COO input

def _coo_of(w, rng, shuffle):
    ri = oracle.csr_to_coo(w.row_ptrs)
    p = rng.permutation(w.nnz) if shuffle else np.arange(w.nnz)
    return ri[p].copy(), w.col_idx[p].copy(), w.values[p].copy()


@pytest.mark.parametrize("name", ["fig14_1", "c2s", "c4s", "c5s"])
@pytest.mark.parametrize("shuffle", [False, True])
def test_coo_to_csr_bitexact(dev, name, shuffle):
    w = synth.fig14_1() if name == "fig14_1" else W(name)
    rng = np.random.default_rng(77)
    ri, ci, v = _coo_of(w, rng, shuffle)
    # duplicates: repeat a few entries (they stay, in input order)
    if w.nnz > 10:
        extra = rng.integers(0, w.nnz, 10)
        ri = np.concatenate([ri, ri[extra]]); ci = np.concatenate([ci, ci[extra]])
        v = np.concatenate([v, v[extra]])
    rp_o, ci_o, v_o = oracle.coo_to_csr(w.num_rows, ri, ci, v)
    t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    rp_d, ci_d, v_d = spmv.coo_to_csr(t(ri), t(ci), t(v), w.num_rows, w.num_cols)
    assert np.array_equal(rp_d.cpu().numpy(), rp_o)
    assert np.array_equal(ci_d.cpu().numpy(), ci_o)
    assert np.array_equal(bits(v_d.cpu().numpy()), bits(v_o))


@pytest.mark.parametrize("num_rows,nnz,hot", [
    (200, 4096 * 3 + 17, 0.0),          # one 8-bit pass, ragged last tile
    (70_000, 1_000_003, 0.0),           # three passes (17-bit rows), ragged tile
    (300_000, 2_500_001, 0.6),          # three passes; 60 % of entries in 5 rows
    (1 << 20, 4096, 0.5),               # fewer entries than one tile, mostly one row
])
def test_coo_to_csr_sort_shapes(dev, num_rows, nnz, hot):
    """The COO -> CSR stable sort at the shapes its passes and tiles take:
    one or three digit passes, a ragged last tile, and runs of equal rows
    that span many 4096-entry tiles (stability across tiles and passes).
    Columns are the entry's input position, so the output columns also show
    the order inside each row; bit-exact against the oracle."""
    rng = np.random.default_rng(num_rows + nnz)
    ri = rng.integers(0, num_rows, nnz).astype(np.int32)
    if hot:
        k = int(hot * nnz)
        ri[rng.permutation(nnz)[:k]] = rng.integers(0, num_rows, 5)[rng.integers(0, 5, k)]
    ci = (np.arange(nnz) % (1 << 30)).astype(np.int32)
    v = rng.standard_normal(nnz).astype(np.float32)
    rp_o, ci_o, v_o = oracle.coo_to_csr(num_rows, ri, ci, v)
    t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    rp_d, ci_d, v_d = spmv.coo_to_csr(t(ri), t(ci), t(v), num_rows, 1 << 30)
    assert np.array_equal(rp_d.cpu().numpy(), rp_o)
    assert np.array_equal(ci_d.cpu().numpy(), ci_o)
    assert np.array_equal(bits(v_d.cpu().numpy()), bits(v_o))


@pytest.mark.parametrize("fmt", ALL_FORMATS)
def test_build_coo_spmv(dev, fmt):
    w = W("c4s")
    rng = np.random.default_rng(3)
    ri, ci, v = _coo_of(w, rng, True)
    t = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    if fmt in ("ell", "ell_xtile"):
        w = W("c2s" if fmt == "ell" else "c3s")
        ri, ci, v = _coo_of(w, rng, True)
    h = spmv.build_coo(fmt, t(ri), t(ci), t(v), w.num_rows, w.num_cols)
    y_ref, bound = oracle.spmv_coo(w.num_rows, ri, ci, v, w.x, w.y)
    assert_rows(run_once(h, t(w.x), t(w.y)), y_ref, bound, f"coo input {fmt}")


def test_coo_bad_row_index(dev):
    t = lambda a: torch.from_numpy(np.asarray(a, np.int32)).to(dev)  # noqa: E731
    for ri, ci, code in (([0, 4], [0, 0], 4), ([0, -1], [0, 0], 4), ([0, 1], [0, 9], 3)):
        assert oracle.validate_coo(4, 4, ri, ci) == code
        with pytest.raises(spmv.SpmvError) as ei:
            spmv.coo_to_csr(t(ri), t(ci), torch.ones(2, device=dev), 4, 4)
        assert ei.value.status == code


# ------------------------------------------------------ full-size workloads

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("fmt", ALL_FORMATS + ["auto"])
def test_full_size_parity(dev, name, fmt):
    """Full-size workloads, every format, every row against the oracle.
    ELL is refused where R * W overflows int32 slots (skewed, power law)."""
    w = W(name)
    Wd = int(np.diff(w.row_ptrs).max())
    print(f"[case] full {name} {fmt} R={w.num_rows} nnz={w.nnz} W={Wd}", flush=True)
    if fmt == "ell" and w.num_rows * Wd > 2**31 - 1:
        expect_refused(fmt, w, dev)
        return
    if fmt == "ell_xtile" and xtile_refused(w.row_ptrs, w.col_idx, w.values):
        expect_refused(fmt, w, dev)
        return
    kw = {"hyb_width": 20} if (fmt == "hyb" and name == "c4") else {}
    h = build(fmt, w, dev, **kw)
    if fmt == "auto":
        # the automatic build's whole decision (selector, x tiles, blocked COO
        # and its slice count) equals the oracle's written-out rule
        f, K, L, S = oracle.select_build(w.row_ptrs, w.col_idx, w.num_cols, spmv.BC_BLOCK_ROWS)
        assert (h.format, h.info["hyb_width"], h.info["lanes_per_row"],
                h.info["col_blocks"]) == (f, K, L, S)
        # the 2-D stencil and the random 5-per-row matrix: ELL; the 3-D
        # stencil: x tiles; skewed and power law (x of 8 / 16 MB): blocked COO
        assert f == {"c1": "ell", "c2": "ell", "c3": "ell_xtile", "c4": "coo_blocked",
                     "c5": "coo_blocked"}[name]
    elif fmt == "coo_blocked":
        # x within 4 MiB slices
        assert h.info["col_blocks"] == {"c1": 1, "c2": 1, "c3": 2, "c4": 2, "c5": 4}[name]
    else:
        assert h.info["col_blocks"] == 1
    _, _, _, x, y0 = to_dev(w, dev)
    y_ref, bound = ref(name)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"full {name}/{fmt}")


@pytest.mark.parametrize("name,fmt", [("c1", "ell"), ("c2", "ell"), ("c3", "ell"),
                                      ("c1", "ell_xtile"), ("c3", "ell_xtile"),
                                      ("c4", "hyb"), ("c4", "jds"), ("c5", "jds"),
                                      ("c5", "coo_segmented"), ("c4", "sell"), ("c5", "sell"),
                                      ("c2", "coo_blocked"), ("c4", "coo_blocked"),
                                      ("c5", "coo_blocked")])
def test_full_size_builders_bitexact(dev, name, fmt):
    w = W(name)
    print(f"[case] full builder {name} {fmt}", flush=True)
    kw = {"hyb_width": 20} if fmt == "hyb" else {}
    h = build(fmt, w, dev, **kw)
    check_builder(h, w)


@pytest.mark.parametrize("name,expect", [("c4", ("hyb", 20)), ("c5", ("csr_merge", 0))])
def test_full_size_selector_unsliced(dev, name, expect):
    """Without x slices the selector picks HYB(20) for the skewed matrix (the
    width the format-choice article found best) and merge CSR for power law."""
    h = build("auto", W(name), dev, col_blocks=1)
    assert (h.format, h.info["hyb_width"]) == expect and h.info["col_blocks"] == 1


# ------------------------------------------------------------- blocked COO

@pytest.mark.parametrize("name", ["c2s", "c4s", "c5s", "c1s"])
@pytest.mark.parametrize("S", [1, 2, 4, 8])
def test_blocked_slice_counts(dev, name, S):
    """Blocked COO with 1, 2, 4 and 8 x slices (slice k's chunks on their own
    XCDs): every array bit-exact against the oracle, y within the row bound,
    and twice in a row y + 2 A x (partials accumulate into y, never overwrite)."""
    w = W(name)
    print(f"[case] blocked {name} S={S}", flush=True)
    h = build("coo_blocked", w, dev, col_blocks=S)
    assert h.format == "coo_blocked" and h.info["col_blocks"] == S
    check_builder(h, w)
    _, _, _, x, y0 = to_dev(w, dev)
    y_ref, bound = ref(name)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"{name} blocked S={S}")
    y = y0.clone()
    h.run(x, y)
    h.run(x, y)
    torch.cuda.synchronize()
    y2 = 2 * (y_ref - w.y.astype(np.float64)) + w.y.astype(np.float64)
    assert_rows(y.cpu().numpy(), y2, 2 * bound, f"{name} blocked S={S} twice")


def _wide_mix():
    """2,000 rows over 10M columns: half the rows keep their columns in a
    narrow band (groups spanning < 2^16 columns), the rest scatter them over
    all of x (groups spanning more: wide groups with full columns)."""
    if "wide_mix" in _cache:
        return _cache["wide_mix"]
    rng = np.random.default_rng(77)
    R, C = 2000, 10_000_000
    lens = rng.integers(1, 9, size=R)
    cols = []
    for r, l in enumerate(lens):
        lo, hi = (5_000_000, 5_030_000) if r % 2 else (0, C)
        cols.append(np.sort(rng.choice(np.arange(lo, hi), l, replace=False)))
    ci = np.concatenate(cols).astype(np.int32)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    _cache["wide_mix"] = synth.Workload("wide_mix", R, C, rp, ci,
                                        rng.uniform(-1, 1, ci.size).astype(np.float32),
                                        rng.uniform(-1, 1, C).astype(np.float32),
                                        rng.uniform(-1, 1, R).astype(np.float32))
    return _cache["wide_mix"]


@pytest.mark.parametrize("S", [1, 8])
def test_blocked_wide_groups(dev, S):
    w = _wide_mix()
    h = build("coo_blocked", w, dev, col_blocks=S)
    assert h.info["wide_groups"] > 0 and h.info["wide_groups"] < h.info["groups"]
    check_builder(h, w)
    y_ref, bound = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"wide groups S={S}")


def test_blocked_hot_rows(dev):
    """Two row blocks over 3M columns; block 0 has 40 rows longer than the hot
    threshold (more than its 32 hot slots; several of equal length, so the
    row-number tie rule decides), block 1 a few, one of them 30,000 long: hot
    rows get per-wave partials, the rest compare-and-swap.  Bit-exact arrays,
    y within the bound."""
    rng = np.random.default_rng(91)
    RB = spmv.BC_BLOCK_ROWS
    R, C = RB + 3616, 3_000_000
    lens = rng.integers(0, 8, size=R)
    long0 = rng.choice(RB, 40, replace=False)
    lens[long0] = rng.choice([100, 150, 150, 200, 300], size=40)
    lens[[RB + 616, RB + 1616, R - 1]] = [30000, 70, 500]
    cols = [np.sort(rng.choice(C, l, replace=False)) if l else np.zeros(0, np.int64) for l in lens]
    ci = np.concatenate(cols).astype(np.int32)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    w = synth.Workload("hot_rows", R, C, rp, ci, rng.uniform(-1, 1, ci.size).astype(np.float32),
                       rng.uniform(-1, 1, C).astype(np.float32),
                       rng.uniform(-1, 1, R).astype(np.float32))
    h = build("coo_blocked", w, dev, col_blocks=1)
    hot = h.array("bc_hot").reshape(-1, h.info["hot_slots"])
    assert (hot[0] >= 0).all() and (hot[1] >= 0).sum() == 3
    check_builder(h, w)
    y_ref, bound = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), y_ref, bound, "hot rows")


@pytest.mark.parametrize("blocks,extra_rows,mode", [(64, 0, "chunk"), (65, 0, "balanced"),
                                                     (65, 11_000, "balanced"), (65, 0, "mixed"),
                                                     (81, 0, "holes")])
def test_blocked_balanced_items(dev, blocks, extra_rows, mode):
    """2 x slices of 2M columns, 2 entries per row.  With 64 row blocks each
    slice's 128 chunks fill its 128 CUs once and stay one chunk per work
    item; with 65 blocks (and with a partial 66th) the 130-odd chunks would
    leave a short second round, so each slice is cut into 128 work items of
    equal cost, chunks split at the items' ends, several chunks per item.
    Mixed: every row's entries in the first slice but one row in 8 with a
    third entry in the second, which is then too small to balance (one chunk
    per item) while the first is balanced.  Holes: 81 blocks, every fifth
    one empty (65 with entries): empty segments inside balanced slices.
    Arrays bit-exact against the
    oracle; y within the row bound, once and twice in a row (the partials
    reset between an item's chunks)."""
    rng = np.random.default_rng(4100 + blocks + extra_rows + (mode == "mixed"))
    R, C = blocks * spmv.BC_BLOCK_ROWS + extra_rows, 2_000_000
    lo = C // 2 if mode == "mixed" else C
    cols = np.sort(rng.integers(0, lo, size=(R, 2)), axis=1)
    cols[:, 1] += cols[:, 0] == cols[:, 1]
    cols = np.minimum(cols, C - 1)
    if mode == "mixed":
        third = np.where(np.arange(R) % 8 == 0, rng.integers(C // 2, C, size=R), -1)
        lens = 2 + (third >= 0)
        ci = np.concatenate([np.concatenate([c, [t]]) if t >= 0 else c
                             for c, t in zip(cols, third)]).astype(np.int32)
        rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    elif mode == "holes":
        keep = (np.arange(R) // spmv.BC_BLOCK_ROWS) % 5 != 4
        ci = cols[keep].reshape(-1).astype(np.int32)
        rp = np.concatenate([[0], np.cumsum(2 * keep)]).astype(np.int32)
    else:
        ci = cols.reshape(-1).astype(np.int32)
        rp = np.arange(0, 2 * R + 1, 2, dtype=np.int32)
    w = synth.Workload("balanced", R, C, rp, ci, rng.uniform(-1, 1, ci.size).astype(np.float32),
                       rng.uniform(-1, 1, C).astype(np.float32),
                       rng.uniform(-1, 1, R).astype(np.float32))
    print(f"[case] blocked items {mode} R={R} nnz={w.nnz}", flush=True)
    h = build("coo_blocked", w, dev)
    assert h.info["col_blocks"] == 2
    items = h.info["work_items"]
    sitem, ichunk = h.array("bc_slice_item"), h.array("bc_item_chunk")
    per_slice = np.diff(sitem).tolist()
    if mode in ("balanced", "holes"):
        assert per_slice == [128, 128] and h.info["num_tiles"] > items
    elif mode == "mixed":
        assert per_slice[0] == 128 and np.diff(ichunk[sitem[1]:]).tolist() == [1] * per_slice[1]
    else:
        assert items == h.info["num_tiles"]
    check_builder(h, w)
    y_ref, bound = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"items {mode} {blocks}+{extra_rows}")
    y = y0.clone()
    h.run(x, y)
    h.run(x, y)
    torch.cuda.synchronize()
    y2 = 2 * (y_ref - w.y.astype(np.float64)) + w.y.astype(np.float64)
    assert_rows(y.cpu().numpy(), y2, 2 * bound, f"items {mode} {blocks}+{extra_rows} twice")


@pytest.mark.parametrize("S", [1, 2])
def test_blocked_scan_runs(dev, S):
    """Every row's entries sit in a column range of their own, so the column
    order of a segment is row order and each group of 64 lanes holds runs of
    one row: lengths 1..64 at every lane offset, runs that cross the 16-lane
    DPP rows (lanes 15/16, 31/32, 47/48) and runs that fill whole groups, plus
    hot rows (longer than 64 * S) whose runs go to per-wave slots.  Groups of
    singletons (the scan skipped) sit beside groups of long runs.  Bit-exact
    arrays, y within the bound."""
    rng = np.random.default_rng(123 + S)
    R = 6000
    lens = rng.integers(1, 65, size=R)
    lens[1000:2000] = 1                                # a stretch of one-entry rows
    lens[rng.choice(R, 50, replace=False)] = rng.integers(64 * S + 1, 400, size=50)
    starts = np.concatenate([[0], np.cumsum(lens + 3)[:-1]])
    C = int(starts[-1] + lens[-1] + 3)
    ci = np.concatenate([np.arange(a, a + l) for a, l in zip(starts, lens)]).astype(np.int32)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    w = synth.Workload("scan_runs", R, C, rp, ci, rng.uniform(-1, 1, ci.size).astype(np.float32),
                       rng.uniform(-1, 1, C).astype(np.float32),
                       rng.uniform(-1, 1, R).astype(np.float32))
    h = build("coo_blocked", w, dev, col_blocks=S)
    assert h.info["wide_groups"] == 0 and (h.array("bc_hot") >= 0).sum() > 0
    check_builder(h, w)
    codes = (h.array("bc_pk") >> 16).reshape(-1, 64)
    real = codes != 0xFFFF
    same = (codes[:, 1:] == codes[:, :-1]) & real[:, 1:]
    assert (~same.any(axis=1)).any() and same.all(axis=1).any()   # both kinds of group
    assert same[:, [14, 30, 46]].any(axis=0).all()                  # runs across DPP rows
    y_ref, bound = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"scan runs S={S}")


@pytest.fixture(scope="module")
def x_past_2_30(dev):
    """x of 2^30 + 1 columns (4 GiB), generated on the device."""
    g = torch.Generator(device=dev)
    g.manual_seed(2030)
    x = torch.rand((1 << 30) + 1, generator=g, device=dev)
    x.mul_(2).sub_(1)
    yield x
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("C,S", [(1 << 30, 1), ((1 << 30) + 1, 1), ((1 << 30) + 1, 8)])
def test_blocked_x_of_2_30_columns(dev, x_past_2_30, C, S):
    """x slices at the edge of 32-bit byte offsets: one slice of exactly 2^30
    columns (gathers up to byte 2^32 - 4 of the slice), one of 2^30 + 1 (the
    64-bit gather path), and 8 slices of the larger x.  Odd rows keep their
    columns in a band below C (narrow groups whose offsets reach the top of
    the slice), even rows scatter them over all of x (wide groups).  y against
    the oracle on the same matrix with its columns renumbered densely (the
    oracle sees the same products in the same row order)."""
    rng = np.random.default_rng(2030 + S + C)
    R = 4096
    lens = rng.integers(1, 17, size=R)
    cols = []
    for r, n in enumerate(lens):
        lo = C - 40_000 if r % 2 else 0
        c = np.sort(rng.choice(C - lo, n, replace=False) + lo)
        cols.append(c)
    cols[1][-1] = C - 1                                   # the last column itself
    ci = np.concatenate(cols).astype(np.int32)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    va = rng.uniform(-1, 1, ci.size).astype(np.float32)
    y0 = rng.uniform(-1, 1, R).astype(np.float32)
    print(f"[case] blocked x of {C} columns, S={S}", flush=True)
    h = spmv.build("coo_blocked", torch.from_numpy(rp).to(dev), torch.from_numpy(ci).to(dev),
                   torch.from_numpy(va).to(dev), C, col_blocks=S)
    assert h.info["col_blocks"] == S and h.info["slice_cols"] == -(-C // S)
    assert 0 < h.info["wide_groups"] < h.info["groups"]
    y = torch.from_numpy(y0).to(dev)
    h.run(x_past_2_30[:C], y)
    torch.cuda.synchronize()
    uniq, local = np.unique(ci, return_inverse=True)
    xl = x_past_2_30[torch.from_numpy(uniq.astype(np.int64)).to(dev)].cpu().numpy()
    y_ref, bound = oracle.spmv_csr(rp, local.astype(np.int32), va, xl, y0)
    assert_rows(y.cpu().numpy(), y_ref, bound, f"x of {C} columns S={S}")
    h.close()


def _slices(w, K):
    """The CSR arrays of the K column slices (entries with column in
    [k*ceil(C/K), (k+1)*ceil(C/K)), row order kept), built with numpy."""
    sc = -(-w.num_cols // K)
    rows = np.repeat(np.arange(w.num_rows), np.diff(w.row_ptrs))
    out = []
    for k in range(K):
        m = (w.col_idx >= k * sc) & (w.col_idx < (k + 1) * sc)
        if not m.any():
            continue
        counts = np.bincount(rows[m], minlength=w.num_rows)
        rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        out.append((rp, w.col_idx[m], w.values[m]))
    return out


@pytest.mark.parametrize("name", ["c2s", "c4s", "c5s", "c3s"])
@pytest.mark.parametrize("fmt", ALL_FORMATS + ["auto"])
def test_col_slices_parity(dev, name, fmt):
    """Every format split into 3 x slices (and auto) still meets the row bound;
    a sliced handle exports only the histogram."""
    w = W(name)
    if fmt == "ell" and name in ("c4s", "c5s"):
        pytest.skip("ELL of a skewed slice is mostly padding")
    if fmt == "ell_xtile" and any(xtile_refused(*sl) for sl in _slices(w, 3)):
        expect_refused(fmt, w, dev, col_blocks=3)
        return
    if fmt == "coo_blocked":
        # its slice count is 1, 2, 4 or 8; 3 is an invalid argument
        with pytest.raises(spmv.SpmvError) as ei:
            build(fmt, w, dev, col_blocks=3)
        assert ei.value.name == "SPMV_ERR_INVALID_ARG"
        h = build(fmt, w, dev, col_blocks=4)
        assert h.info["col_blocks"] == 4 and h.info["slice_cols"] == -(-w.num_cols // 4)
        check_blocked(h, w)
        _, _, _, x, y0 = to_dev(w, dev)
        assert_rows(run_once(h, x, y0), *ref(name), f"{name}/{fmt} 4 slices")
        return
    h = build(fmt, w, dev, col_blocks=3)
    assert h.info["col_blocks"] == 3
    assert h.info["slice_cols"] == -(-w.num_cols // 3)
    assert not h.has_array("col_idx") and not h.has_array("ell_col")
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), *ref(name), f"{name}/{fmt} 3 slices")


@pytest.mark.parametrize("name", ["c4s", "c5s", "c2s"])
@pytest.mark.parametrize("k", [2, 4, 8])
def test_merge_slices_in_one_launch(dev, name, k):
    """Merge-CSR slices whose count divides 8 run in one launch, each slice on
    its own XCDs, with every row's sum added to y atomically; y meets the row
    bound, and so does a y that already holds data (accumulation, not
    overwrite)."""
    w = W(name)
    h = build("csr_merge", w, dev, col_blocks=k)
    assert h.info["col_blocks"] == k and h.format == "csr_merge"
    _, _, _, x, y0 = to_dev(w, dev)
    y_ref, bound = ref(name)
    assert_rows(run_once(h, x, y0), y_ref, bound, f"{name} merge {k} slices")
    # twice in a row: y + 2 A x
    y = y0.clone()
    h.run(x, y)
    h.run(x, y)
    torch.cuda.synchronize()
    y2 = 2 * (y_ref - w.y.astype(np.float64)) + w.y.astype(np.float64)
    assert_rows(y.cpu().numpy(), y2, 2 * bound, f"{name} merge {k} slices twice")


def test_merge_slices_uneven_and_empty(dev):
    """Columns crowded into the first quarter of x: with 4 slices, slice 0
    holds most entries and the others few (uneven tile counts; blocks of the
    short slices exit early); with 8 slices some slices are empty and are
    dropped, and a count that no longer divides 8 runs one launch per slice.
    Every case meets the row bound."""
    rng = np.random.default_rng(404)
    w = synth.small_random(rng, 100_000, 400_000, max_len=20, empty_frac=0.1)
    # squeeze 90 % of the columns into [0, 100000)
    squeeze = rng.random(w.nnz) < 0.9
    w.col_idx = np.where(squeeze, w.col_idx % 100_000, w.col_idx).astype(np.int32)
    w.col_idx[:200] = 399_999            # keep the last slice non-empty for k = 4
    yref, bound = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    rp, ci, v, x, y0 = to_dev(w, dev)
    for k in (2, 4, 8, 16):
        h = spmv.build("csr_merge", rp, ci, v, w.num_cols, col_blocks=k)
        assert_rows(run_once(h, x, y0), yref, bound, f"uneven slices k={k}")


@pytest.mark.parametrize("fmt", ["auto", "csr_merge", "coo_segmented", "csr_vector", "jds", "hyb"])
def test_full_size_power_law_slices(dev, fmt):
    w = W("c5")
    h = build(fmt, w, dev, col_blocks=8)
    _, _, _, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), *ref("c5"), f"c5/{fmt} 8 slices")


@pytest.mark.parametrize("name", ["c1s", "c2s", "c4s", "c5s"])
def test_empirical_selector(dev, name):
    """The tuned handle is the fastest built candidate, computes y within the
    bound, and the candidates that cannot exist are reported as refused."""
    w = W(name)
    rp, ci, v, x, y0 = to_dev(w, dev)
    h, rep = spmv.build_tuned(rp, ci, v, w.num_cols, runs=3)
    built = [e for e in rep if e["status"] == "SPMV_OK"]
    chosen = [e for e in rep if e["chosen"]]
    assert len(chosen) == 1 and chosen[0]["us"] == min(e["us"] for e in built)
    assert h.format == chosen[0]["format"] and h.info["col_blocks"] == chosen[0]["col_blocks"]
    assert {e["format"] for e in rep} >= set(ALL_FORMATS)
    if name in ("c5s",):
        assert any(e["format"] == "ell" and e["status"] == "SPMV_ERR_TOO_LARGE" for e in rep)
    assert_rows(run_once(h, x, y0), *ref(name), f"tuned {name}")


def test_empirical_selector_mask(dev):
    w = W("c2s")
    rp, ci, v, _, _ = to_dev(w, dev)
    h, rep = spmv.build_tuned(rp, ci, v, w.num_cols, formats=["csr_scalar", "jds"], runs=2)
    assert {e["format"] for e in rep} == {"csr_scalar", "jds"}
    assert h.format in ("csr_scalar", "jds")


@pytest.mark.parametrize("fmt", ["ell", "csr_vector", "csr_merge", "sell", "ell_xtile"])
@pytest.mark.parametrize("name", ["c1s", "c1"])
def test_conjugate_gradient(dev, fmt, name):
    """CG on the 5-point Laplacian (symmetric positive definite) recovers a
    known solution: b = A x_true (fp64 oracle product), x0 = 0.  The final
    true residual is checked with the oracle's exact SpMV."""
    w = W(name)
    x_true = w.x.astype(np.float64)
    b, _ = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, np.zeros(w.num_rows, np.float32))
    b32 = b.astype(np.float32)
    h = build(fmt, w, dev)
    x = torch.zeros(w.num_rows, device=dev)
    rtol = 1e-5
    iters, rel = h.cg(torch.from_numpy(b32).to(dev), x, max_iter=5000, rtol=rtol)
    assert rel <= rtol and 0 < iters < 5000
    xs = x.cpu().numpy()
    ax, _ = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, xs, -b32)   # A x - b in fp64
    assert np.linalg.norm(ax) / np.linalg.norm(b32.astype(np.float64)) <= 10 * rtol
    # condition number of the n x n Laplacian ~ (2n/pi)^2
    n = int(round(np.sqrt(w.num_rows)))
    kappa = (2 * n / np.pi) ** 2
    assert np.max(np.abs(xs - x_true)) <= 10 * kappa * rtol


def test_conjugate_gradient_rejects_rectangular(dev):
    rng = np.random.default_rng(1)
    w = synth.small_random(rng, 5, 7, max_len=3)
    h = build("csr_scalar", w, dev)
    with pytest.raises(spmv.SpmvError):
        h.cg(torch.zeros(5, device=dev), torch.zeros(5, device=dev))


def _cg_rhs(w):
    """b = A x_true rounded to fp32 (the oracle's fp64 product)."""
    b, _ = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, np.zeros(w.num_rows, np.float32))
    return b.astype(np.float32)


@pytest.mark.parametrize("fmt", ["ell", "csr_merge", "sell", "sliced"])
@pytest.mark.parametrize("k", [1, 2, 5, 8, 13, 40])
def test_cg_iterates_match_oracle(dev, fmt, k):
    """After exactly k iterations (rtol 0) the device's x equals the oracle's
    fp64 CG iterate within k * kappa * 2^-24 * max|x| (k fp32 steps, each
    rounding error amplified at most by the condition number kappa)."""
    w = W("c1s")
    b32 = _cg_rhs(w)
    h = build("csr_merge", w, dev, col_blocks=2) if fmt == "sliced" else build(fmt, w, dev)
    x = torch.zeros(w.num_rows, device=dev)
    iters, _ = h.cg(torch.from_numpy(b32).to(dev), x, max_iter=k, rtol=0.0)
    assert iters == k
    xo, ko, _ = oracle.cg(w.row_ptrs, w.col_idx, w.values, b32.astype(np.float64),
                          max_iter=k, rtol=0.0)
    assert ko == k
    n = int(round(np.sqrt(w.num_rows)))
    kappa = (2 * (n + 1) / np.pi) ** 2
    tol = k * kappa * 2.0**-24 * np.max(np.abs(xo))
    err = np.max(np.abs(x.cpu().numpy().astype(np.float64) - xo))
    print(f"cg {fmt} k={k}: max err {err:.3e} tol {tol:.3e}")
    assert err <= tol


@pytest.mark.parametrize("name", ["c1s", "c1"])
def test_cg_iteration_count_matches_oracle(dev, name):
    """To rtol 1e-5 the device stops at the first multiple of 8 at or past the
    oracle's iteration count, give or take one check for fp32 rounding."""
    w = W(name)
    b32 = _cg_rhs(w)
    h = build("ell", w, dev)
    x = torch.zeros(w.num_rows, device=dev)
    iters, rel = h.cg(torch.from_numpy(b32).to(dev), x, max_iter=5000, rtol=1e-5)
    _, ko, _ = oracle.cg(w.row_ptrs, w.col_idx, w.values, b32.astype(np.float64),
                         max_iter=5000, rtol=1e-5)
    print(f"cg {name}: device {iters} iterations, oracle {ko}")
    ceil8 = -(-ko // 8) * 8
    assert iters % 8 == 0 and ceil8 - 8 <= iters <= ceil8 + 8


def test_cg_deterministic_with_ell(dev):
    """ELL's SpMV and the block-ordered fp64 dot products have a fixed summation
    order: two solves give bit-identical x."""
    w = W("c1s")
    b = torch.from_numpy(_cg_rhs(w)).to(dev)
    h = build("ell", w, dev)
    xs = []
    for _ in range(2):
        x = torch.zeros(w.num_rows, device=dev)
        h.cg(b, x, max_iter=50, rtol=0.0)
        xs.append(x.cpu().numpy())
    assert np.array_equal(xs[0].view(np.uint32), xs[1].view(np.uint32))


def test_cg_degenerate_cases(dev):
    w = W("c1s")
    h = build("ell", w, dev)
    b = torch.from_numpy(_cg_rhs(w)).to(dev)
    # max_iter 0: x untouched, residual of the start reported
    x = torch.full((w.num_rows,), 0.5, device=dev)
    iters, rel = h.cg(b, x, max_iter=0, rtol=1e-6)
    assert iters == 0 and rel > 0 and torch.all(x == 0.5)
    # b = 0 from x = 0: already solved
    x = torch.zeros(w.num_rows, device=dev)
    iters, rel = h.cg(torch.zeros_like(b), x, max_iter=100, rtol=1e-6)
    assert iters == 0 and rel == 0.0 and not torch.any(x)
    # 1 x 1 system: one step gives b / a
    rp = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    ci = torch.tensor([0], dtype=torch.int32, device=dev)
    v = torch.tensor([4.0], device=dev)
    h1 = spmv.build("csr_scalar", rp, ci, v, 1)
    x = torch.zeros(1, device=dev)
    iters, rel = h1.cg(torch.tensor([2.0], device=dev), x, max_iter=100, rtol=1e-6)
    assert x.item() == 0.5 and rel == 0.0 and iters == 8   # checked after 8 steps
    # empty matrix
    h0 = spmv.build("ell", torch.zeros(1, dtype=torch.int32, device=dev),
                    torch.zeros(0, dtype=torch.int32, device=dev),
                    torch.zeros(0, device=dev), 0)
    assert h0.cg(torch.zeros(0, device=dev), torch.zeros(0, device=dev)) == (0, 0.0)


def _ragged_narrow():
    """2^20 rows of 0..8 random entries (about 11 % empty): the 4-rows-per-lane
    ELL path (R % 4 == 0, narrow width, large grid) with ragged rows."""
    key = ("ragged_narrow",)
    if key not in _cache:
        rng = np.random.default_rng(2024)
        w = synth.small_random(rng, 1 << 20, 1 << 20, max_len=8, empty_frac=0.0)
        _cache[key] = (w, oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y))
    return _cache[key]


@pytest.mark.parametrize("fmt,kw", [("ell", {}), ("hyb", {"hyb_width": 4}), ("hyb", {"hyb_width": 8})])
def test_ell_four_rows_per_lane_ragged(dev, fmt, kw):
    w, (yref, bound) = _ragged_narrow()
    assert int(np.diff(w.row_ptrs).max()) == 8 and (np.diff(w.row_ptrs) == 0).any()
    rp, ci, v, x, y0 = to_dev(w, dev)
    h = spmv.build(fmt, rp, ci, v, w.num_cols, **kw)
    yg = run_once(h, x, y0)
    n_bad, first, worst = oracle.check(yg, yref, bound)
    assert n_bad == 0, (first, worst)
    # empty rows come back bit-identical
    empty = np.diff(w.row_ptrs) == 0
    assert np.array_equal(yg[empty].view(np.uint32), w.y[empty].view(np.uint32))


def _ragged_wide():
    """2^20 rows of 0..40 random entries: the 4-rows-per-lane ELL path at widths
    past one 4-slot step, with ragged and empty rows."""
    key = ("ragged_wide",)
    if key not in _cache:
        rng = np.random.default_rng(4048)
        w = synth.small_random(rng, 1 << 20, 1 << 20, max_len=40, empty_frac=0.05)
        _cache[key] = (w, oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y))
    return _cache[key]


@pytest.mark.parametrize("fmt,kw", [("ell", {}), ("hyb", {"hyb_width": 12}),
                                    ("hyb", {"hyb_width": 20})])
def test_ell_four_rows_per_lane_wide(dev, fmt, kw):
    w, (yref, bound) = _ragged_wide()
    lens = np.diff(w.row_ptrs)
    assert int(lens.max()) == 40 and (lens == 0).any()
    rp, ci, v, x, y0 = to_dev(w, dev)
    h = spmv.build(fmt, rp, ci, v, w.num_cols, **kw)
    yg = run_once(h, x, y0)
    n_bad, first, worst = oracle.check(yg, yref, bound)
    assert n_bad == 0, (first, worst)
    empty = lens == 0
    assert np.array_equal(yg[empty].view(np.uint32), w.y[empty].view(np.uint32))


@pytest.mark.parametrize("max_len,empty,run", [(2, 0.0, 4), (8, 0.0, 8), (14, 0.1, 16),
                                               (60, 0.05, 32)])
def test_coo_atomic_runs(dev, max_len, empty, run):
    """The COO atomic kernel takes RUN consecutive entries per lane, RUN chosen
    from mean + one standard deviation of the row lengths; each choice on a
    ragged matrix whose entry count is not a multiple of RUN."""
    rng = np.random.default_rng(31 + max_len)
    w = synth.small_random(rng, 200_003, 150_001, max_len=max_len, empty_frac=empty)
    lens = np.diff(w.row_ptrs).astype(np.float64)
    spread = lens.mean() + lens.std()
    expect = 4
    while expect < 32 and expect <= spread:
        expect *= 2
    assert expect == run and w.nnz % run != 0
    yref, bound = oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
    h = build("coo_atomic", w, dev)
    rp, ci, v, x, y0 = to_dev(w, dev)
    assert_rows(run_once(h, x, y0), yref, bound, f"coo_atomic run {run}")


@pytest.mark.parametrize("name", ["c3s", "c4s", "c3"])
def test_csr_scalar_staged_rows_match_direct_loads(dev, name):
    """On matrices whose rows average more than 8 entries with under 1 % longer
    than 32, CSR scalar stages each wave's rows through LDS; each row's sum is
    taken in the same order as the direct-load kernel (which CSR vector with
    one lane per row runs), so y is bit-identical."""
    w = W(name)
    lens = np.diff(w.row_ptrs)
    assert lens.mean() > 8 and 100 * (lens > 32).sum() < len(lens)
    rp, ci, v, x, y0 = to_dev(w, dev)
    ys = spmv.build("csr_scalar", rp, ci, v, w.num_cols)
    yd = spmv.build("csr_vector", rp, ci, v, w.num_cols, lanes=1)
    a, b = run_once(ys, x, y0), run_once(yd, x, y0)
    assert np.array_equal(bits(a), bits(b))
    yref, bound = ref(name)
    assert_rows(a, yref, bound, f"csr_scalar staged {name}")


def test_ell_unaligned_y_takes_the_row_per_lane_path(dev):
    """y at a 4-byte offset (not 16-byte aligned): the launcher falls back to
    one row per lane; results are the same."""
    w, (yref, bound) = _ragged_narrow()
    rp, ci, v, x, y0 = to_dev(w, dev)
    h = spmv.build("ell", rp, ci, v, w.num_cols)
    buf = torch.zeros(w.num_rows + 1, device=dev)
    y = buf[1:]
    y.copy_(y0)
    assert y.data_ptr() % 16 != 0
    h.run(x, y)
    torch.cuda.synchronize()
    n_bad, first, worst = oracle.check(y.cpu().numpy(), yref, bound)
    assert n_bad == 0, (first, worst)
    assert buf[0].item() == 0.0


@pytest.mark.parametrize("fmt", ["ell", "sell", "sliced"])
def test_cg_graph_replays_match_eager(dev, fmt, monkeypatch):
    """From 16 iterations on, CG replays one captured 8-iteration graph per
    batch, with host synchronisation and reads between replays.  After every
    number of replays tried, x equals the eager launches' x: bit for bit for
    formats with a fixed summation order, else within k*kappa*2^-24*max|x|."""
    w = W("c1s")
    b = torch.from_numpy(_cg_rhs(w)).to(dev)
    h = build("csr_merge", w, dev, col_blocks=2) if fmt == "sliced" else build(fmt, w, dev)
    n = int(round(np.sqrt(w.num_rows)))
    kappa = (2 * (n + 1) / np.pi) ** 2
    for batches in (2, 3, 5):
        k = 8 * batches
        xs = {}
        for mode in ("1", "0"):
            monkeypatch.setenv("SPMV_CG_GRAPH", mode)
            x = torch.zeros(w.num_rows, device=dev)
            iters, _ = h.cg(b, x, max_iter=k, rtol=0.0)
            assert iters == k
            xs[mode] = x.cpu().numpy()
        if fmt == "sliced":
            tol = k * kappa * 2.0**-24 * np.max(np.abs(xs["0"]))
            assert np.max(np.abs(xs["1"] - xs["0"])) <= tol, batches
        else:
            assert np.array_equal(xs["1"].view(np.uint32), xs["0"].view(np.uint32)), batches


@pytest.mark.parametrize("name", ["c1s", "c1"])
@pytest.mark.parametrize("k", [1, 5, 16, 40])
def test_cg_fused_ell_iteration_matches_four_launches(dev, name, k, monkeypatch):
    """On an ELL handle CG runs two launches per iteration (direction, SpMV
    and p.Ap fused); the arithmetic is the four-launch iteration's, so after k
    iterations (eager below 16, graph replays from 16) x is bit-identical with
    SPMV_CG_FUSED=0."""
    w = W(name)
    b = torch.from_numpy(_cg_rhs(w)).to(dev)
    h = build("ell", w, dev)
    assert h.format == "ell"
    xs = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("SPMV_CG_FUSED", mode)
        x = torch.zeros(w.num_rows, device=dev)
        iters, rel = h.cg(b, x, max_iter=k, rtol=0.0)
        assert iters == k
        xs[mode] = (x.cpu().numpy(), rel)
    assert np.array_equal(xs["1"][0].view(np.uint32), xs["0"][0].view(np.uint32))
    assert xs["1"][1] == xs["0"][1]


def _spd27(n):
    """The 27-point structure on an n^3 grid with diagonal 26 and off-diagonals
    -1: symmetric, diagonally dominant (strictly on the faces), irreducible,
    so positive definite; ELL width 27."""
    w = synth.stencil27(n)
    rows = oracle.csr_to_coo(w.row_ptrs)
    w.values = np.where(w.col_idx == rows, 26.0, -1.0).astype(np.float32)
    return w


@pytest.mark.parametrize("k", [3, 16])
def test_cg_fused_ell_wide_rows(dev, k, monkeypatch):
    """Rows wider than the fused step's 8 preloaded slots (width 27): the fused
    iteration stays bit-identical to the four launches, and after k steps x
    matches the oracle's CG iterate within k * kappa * 2^-24 * max|x|, kappa
    from the operator's extreme eigenvalues (scipy, fp64)."""
    n = 16
    w = _spd27(n)
    b32 = _cg_rhs(w)
    b = torch.from_numpy(b32).to(dev)
    h = build("ell", w, dev)
    assert h.format == "ell" and h.info["ell_width"] == 27
    xs = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("SPMV_CG_FUSED", mode)
        x = torch.zeros(w.num_rows, device=dev)
        iters, _ = h.cg(b, x, max_iter=k, rtol=0.0)
        assert iters == k
        xs[mode] = x.cpu().numpy()
    assert np.array_equal(xs["1"].view(np.uint32), xs["0"].view(np.uint32))
    xo, ko, _ = oracle.cg(w.row_ptrs, w.col_idx, w.values, b32.astype(np.float64),
                          max_iter=k, rtol=0.0)
    assert ko == k
    import scipy.sparse as sp
    import scipy.sparse.linalg as sl
    a = sp.csr_matrix((w.values.astype(np.float64), w.col_idx, w.row_ptrs))
    lo = sl.eigsh(a, k=1, which="SA", return_eigenvectors=False)[0]
    hi = sl.eigsh(a, k=1, which="LA", return_eigenvectors=False)[0]
    assert lo > 0
    tol = k * (hi / lo) * 2.0**-24 * np.max(np.abs(xo))
    assert np.max(np.abs(xs["1"].astype(np.float64) - xo)) <= tol


@pytest.mark.parametrize("grid", [512, 640])
@pytest.mark.parametrize("k", [5, 16])
def test_cg_ell_at_and_past_the_fused_size(dev, grid, k, monkeypatch):
    """Laplacians of 262,144 rows (the largest ELL handle that takes the fused
    iteration: 1,024 blocks of partials) and 409,600 rows (four launches with
    grid-stride vector kernels): x is the same with SPMV_CG_FUSED=0, bit for
    bit, and matches the oracle's CG iterate within k * kappa * 2^-24 * max|x|."""
    key = ("lap", grid)
    if key not in _cache:
        _cache[key] = synth.laplacian2d(grid)
    w = _cache[key]
    b32 = _cg_rhs(w)
    b = torch.from_numpy(b32).to(dev)
    h = build("ell", w, dev)
    assert h.format == "ell"
    xs = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("SPMV_CG_FUSED", mode)
        x = torch.zeros(w.num_rows, device=dev)
        iters, rel = h.cg(b, x, max_iter=k, rtol=0.0)
        assert iters == k
        xs[mode] = (x.cpu().numpy(), rel)
    assert np.array_equal(xs["1"][0].view(np.uint32), xs["0"][0].view(np.uint32))
    assert xs["1"][1] == xs["0"][1]
    xo, ko, _ = oracle.cg(w.row_ptrs, w.col_idx, w.values, b32.astype(np.float64),
                          max_iter=k, rtol=0.0)
    assert ko == k
    kappa = (2 * (grid + 1) / np.pi) ** 2
    tol = k * kappa * 2.0**-24 * np.max(np.abs(xo))
    assert np.max(np.abs(xs["1"][0].astype(np.float64) - xo)) <= tol


@pytest.mark.parametrize("fmt", ALL_FORMATS + ["sliced"])
def test_run_captured_in_a_graph(dev, fmt):
    """spmv_run allocates, sets and synchronises nothing, so a caller can capture
    it in a HIP graph (here torch's).  The graph is replayed 1..4 times, with
    eager work and host reads between replays; after each, y (accumulating
    y += A x) equals the same number of eager runs: bit for bit for the formats
    with a fixed summation order, else within k times the row bound."""
    name = "c3s" if fmt == "ell_xtile" else "c2s"
    w = W(name)
    rp, ci, v, x, y0 = to_dev(w, dev)
    kw = {"col_blocks": 3} if fmt == "sliced" else {}
    h = spmv.build("csr_merge" if fmt == "sliced" else fmt, rp, ci, v, w.num_cols, **kw)
    _, bound = ref(name)
    y_g = y0.clone()
    y_e = y0.clone()
    h.run(x, y_g)                       # warm-up outside the capture, then undo it
    y_g.copy_(y0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.run(x, y_g)
    torch.cuda.synchronize()
    assert torch.equal(y_g, y0)         # capturing ran nothing
    for k in range(1, 5):
        g.replay()
        h.run(x, y_e)
        junk = torch.ones(1 << 20, device=dev).sum()   # eager work between replays
        torch.cuda.synchronize()
        assert junk.item() == float(1 << 20)
        a, b = y_g.cpu().numpy(), y_e.cpu().numpy()
        if fmt in DETERMINISTIC:
            assert np.array_equal(bits(a), bits(b)), (fmt, k)
        else:
            err = np.abs(a.astype(np.float64) - b)
            assert np.all(err <= 2e-5 * k * bound), (fmt, k, float(np.max(err / bound)))
    del g


def test_build_destroy_cycles_release_device_memory(dev):
    """Handles own their device arrays and free them on destroy; builders free
    their scratch: 30 build/run/destroy cycles over every format leave the
    device's free memory where it was."""
    w = W("c2s")
    rp, ci, v, x, y0 = to_dev(w, dev)

    formats = [f for f in ALL_FORMATS if f != "ell_xtile"] + ["ell_xtile_c3s"]
    w3 = W("c3s")
    rp3, ci3, v3, x3, y3 = to_dev(w3, dev)

    def cycle(i):
        fmt = formats[i % len(formats)]
        if fmt == "ell_xtile_c3s":   # the x-tile format needs a banded matrix
            h = spmv.build("ell_xtile", rp3, ci3, v3, w3.num_cols)
            y = y3.clone()
            h.run(x3, y)
            h.close()
            return
        h = spmv.build(fmt, rp, ci, v, w.num_cols, col_blocks=2 if i % 3 == 0 else 0)
        y = y0.clone()
        h.run(x, y)
        h.close()

    # one pass first: the runtime loads each kernel's code and sets up its own
    # pools on first use
    for i in range(2 * len(ALL_FORMATS)):
        cycle(i)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free0, _ = torch.cuda.mem_get_info()
    for i in range(30):
        cycle(i)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 >= free0 - (2 << 20), (free0, free1)


def test_concurrent_host_threads_and_streams(dev):
    """Five host threads each build a handle and run it 20 times on their own
    stream (ctypes releases the GIL during library calls); every result is
    checked against the oracle."""
    import threading
    names = ["c1s", "c2s", "c3s", "c4s", "c5s"]
    fmts = ["ell", "csr_merge", "sell", "hyb", "coo_blocked"]
    results, errors = {}, []
    inputs = {n: to_dev(W(n), dev) for n in names}
    torch.cuda.synchronize()   # the copies above ran on the default stream

    def work(name, fmt):
        try:
            w = W(name)
            rp, ci, v, x, y0 = inputs[name]
            st = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(st):
                h = spmv.build(fmt, rp, ci, v, w.num_cols, stream=st)
                for _ in range(20):
                    y = y0.clone()
                    h.run(x, y, stream=st)
                st.synchronize()
                results[name] = y.cpu().numpy()
                h.close()
        except Exception as e:   # reported below
            errors.append((name, fmt, repr(e)))

    threads = [threading.Thread(target=work, args=a) for a in zip(names, fmts)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for name in names:
        yref, bound = ref(name)
        n_bad, first, worst = oracle.check(results[name], yref, bound)
        assert n_bad == 0, (name, first, worst)
