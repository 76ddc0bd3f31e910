"""The largest matrix the C ABI accepts: nnz = 2^31 - 1 = INT32_MAX, 2^26 rows of
32 entries (the last of 31), columns spread over all of x (synth.BandMatrix).

Every format that fits int32 slots (and blocked COO, whose slot indices are 64-bit)
is built on the device and its y is checked
against the oracle on 4,000 sampled rows (plus the first and last rows and the
middle), to the same row bound as every other parity test.  ELL (2^31 slots)
and sectioned ELL are refused with SPMV_ERR_TOO_LARGE, and an automatic build
falls through to CSR vector.  COO -> CSR is checked on a scrambled COO copy of
the whole matrix: row pointers entirely, column order of sampled rows bit-exact.
The arrays (17 GB per copy) are generated on the device; the sampled rows'
entries come from the generator on the host.
"""
import numpy as np
import pytest

import oracle
from spmv_storage_formats_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import spmv_storage_formats_amd as spmv  # noqa: E402

N_SAMPLES = 4000


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spmv.load_library()
    dev = torch.device("cuda:0")
    m = synth.max_band()
    R = m.num_rows
    print(f"max-size matrix: {R} rows, nnz {m.nnz}", flush=True)
    rp, ci, v = m.csr_tensors(torch, dev)
    x = torch.from_numpy(m.x).to(dev)
    y0 = torch.from_numpy(m.y).to(dev)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 2, R // 2, R - 2, R - 1],
                                     rng.integers(0, R, N_SAMPLES)])).astype(np.int64)
    ent = [m.row(int(r)) for r in rows]
    srp = np.concatenate([[0], np.cumsum([len(c) for c, _ in ent])]).astype(np.int32)
    sci = np.concatenate([c for c, _ in ent])
    sva = np.concatenate([a for _, a in ent])
    yref, bound = oracle.spmv_csr(srp, sci, sva, m.x, m.y[rows])
    torch.cuda.synchronize()
    yield {"m": m, "dev": dev, "rp": rp, "ci": ci, "v": v, "x": x, "y0": y0, "rows": rows,
           "rows_t": torch.from_numpy(rows).to(dev), "yref": yref, "bound": bound,
           "ent": ent}
    del rp, ci, v, x, y0
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,kw", [("csr_scalar", {}), ("csr_vector", {}), ("csr_merge", {}),
                                    ("coo_segmented", {}), ("coo_atomic", {}),
                                    ("hyb", {"hyb_width": 31}), ("jds", {}), ("coo_blocked", {}),
                                    ("auto", {})])
def test_max_size_parity(big, fmt, kw):
    b = big
    print(f"max-size {fmt}", flush=True)
    h = spmv.build(fmt, b["rp"], b["ci"], b["v"], b["m"].num_rows, **kw)
    if fmt == "auto":
        assert h.format == "csr_vector" and h.info["lanes_per_row"] == 32
    if fmt == "hyb":
        assert h.info["tail_nnz"] == b["m"].num_rows - 1
    if fmt == "coo_blocked":
        # 2^26 rows in 2048 blocks, x of 256 MiB in 8 slices; slots past 2^31
        assert h.info["col_blocks"] == 8 and h.info["groups"] * 64 >= b["m"].nnz
    y = b["y0"].clone()
    h.run(b["x"], y)
    yg = y[b["rows_t"]].cpu().numpy()
    h.close()
    del y
    n_bad, first, worst = oracle.check(yg, b["yref"], b["bound"])
    assert n_bad == 0, (fmt, first, worst)


@pytest.mark.parametrize("fmt", ["ell", "sell"])
def test_max_size_padded_formats_refused(big, fmt):
    b = big
    with pytest.raises(spmv.SpmvError) as e:
        spmv.build(fmt, b["rp"], b["ci"], b["v"], b["m"].num_rows)
    assert e.value.name == "SPMV_ERR_TOO_LARGE"


def test_max_size_coo_to_csr(big):
    """COO input in the order i -> entry (i * a) mod nnz (a bijection: nnz = 2^31 - 1
    is prime), converted on the device: row pointers equal the generator's, and
    inside each sampled row the entries keep their COO input order (stable)."""
    b = big
    m, dev = b["m"], b["dev"]
    N, R, a = m.nnz, m.num_rows, 48271
    print("max-size coo_to_csr", flush=True)
    lens = torch.full((R,), m.per_row, dtype=torch.int32, device=dev)
    lens[-1] -= 1
    row_of = torch.repeat_interleave(torch.arange(R, dtype=torch.int32, device=dev), lens)
    perm = (torch.arange(N, dtype=torch.int64, device=dev) * a) % N
    ri = row_of[perm]
    del row_of
    ci = b["ci"][perm]
    va = b["v"][perm]
    del perm
    rp2, ci2, va2 = spmv.coo_to_csr(ri, ci, va, R, R)
    del ri, ci, va
    assert torch.equal(rp2, b["rp"])
    ainv = pow(a, -1, N)
    rp_h = b["rp"][b["rows_t"]].cpu().numpy().astype(np.int64)
    for k, r in enumerate(b["rows"][:500]):
        cols, vals = b["ent"][k]
        j = rp_h[k] + np.arange(len(cols), dtype=np.int64)      # generator positions
        order = np.argsort((j * ainv) % N)                       # COO input positions
        s = int(rp_h[k])
        got_c = ci2[s:s + len(cols)].cpu().numpy()
        got_v = va2[s:s + len(cols)].cpu().numpy()
        assert np.array_equal(got_c, cols[order]), r
        assert np.array_equal(got_v.view(np.uint32), vals[order].view(np.uint32)), r
    del rp2, ci2, va2
    torch.cuda.empty_cache()
