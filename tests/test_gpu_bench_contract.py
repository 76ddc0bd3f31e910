"""bench.py's one-line JSON result on the GPU: the fields and their relations
(the default run -- the power-law headline plus one entry per other workload --
with shortened timing and CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def line():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "4",
                        "--warmup", "1", "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=400, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    out = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(out) == 1, p.stdout[-2000:]
    return json.loads(out[0])


def _alg(R, C, nnz):
    # algorithmic bytes: 8 per nonzero, row pointers, x once, y read and written
    return 8 * nnz + 4 * (R + 1) + 4 * C + 8 * R


def test_contract_fields(line):
    d = line
    assert d["metric"].startswith("SpMV GFLOP/s") and d["unit"] == "GFLOP/s"
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["dtype"] == "f32"
    assert d["data"].startswith("synthetic")
    cfg = d["config"]
    # the headline is the largest workload, the power-law matrix
    assert cfg["workload"].startswith("power_law_4M")
    assert (cfg["rows"], cfg["cols"]) == (4_000_000, 4_000_000) and cfg["nnz"] > 60_000_000
    assert cfg["format"] == "coo_blocked" and cfg["col_blocks"] == 4
    # value = 2 nnz / mean step time
    assert d["value"] > 0
    assert abs(d["value"] - 2 * cfg["nnz"] / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]


def test_roofline_fields(line):
    r, cfg = line["roofline"], line["config"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["bytes_per_launch_alg"] == _alg(cfg["rows"], cfg["cols"], cfg["nnz"])
    assert abs(r["achieved"] - r["bytes_per_launch_alg"] / (line["ms_per_step"] * 1e-3) / 1e9) \
        <= 0.01 * r["achieved"]
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-3
    assert 0 < r["frac"] < 1
    # traffic and the profiled duration come from the committed summaries, or
    # are null when the kernel sources changed since they were taken
    assert r["traffic"] is None or (isinstance(r["traffic"], int) and r["traffic"] > 0)
    assert (r["profiled_kernel_us"] is None) == (r["traffic"] is None)


def test_every_workload_has_an_entry(line):
    c = line["configs"]
    assert set(c) == {"c1", "c2", "c3", "c4", "c5"}
    expect = {"c1": "ell", "c2": "ell", "c3": "ell_xtile", "c4": "coo_blocked",
              "c5": "coo_blocked"}
    for name, e in c.items():
        assert e["format"] == expect[name], name
        assert e["alg_bytes"] == _alg(e["rows"], e["cols"], e["nnz"])
        us = e["us_mean"]
        assert abs(e["frac_by_events"] - e["alg_bytes"] / (us * 1e-6) / 1e9 / 8000) <= 1e-3
        assert e["worst_err_over_bound"] <= 1.0
    # the configured HYB with ELL width 20 beside the skewed matrix's format
    assert c["c4"]["hyb_width20"]["format"] == "hyb"
    # every format on the headline matrix: built and checked, or refused
    f = c["c5"]["formats"]
    assert f["ell"] == {"refused": "SPMV_ERR_TOO_LARGE"}
    assert all("us_median" in v or "refused" in v for v in f.values())


def test_device_rates(line):
    g = line["device_rates"]["gather"]["rates"]
    # gathers that share cache lines run faster than random ones
    assert g["x2MiB_sorted_8_per_line"]["g_per_s"] > g["x2MiB_random"]["g_per_s"]
    assert {f"x{m}MiB_random" for m in (2, 4, 8, 16)} <= set(g)
    lds = line["device_rates"]["lds"]
    assert set(lds) == {"lds_float_atomic_add", "cas_float_add", "lds_integer_atomic_add"}


def test_cpu_baseline_fields(line):
    c = line["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "GFLOP/s" and c["cores"] == 1
    assert c["value"] > 0 and "full passes" in c["sample"]
    o = c["openmp"]
    assert o["kind"] == "openmp_csr" and o["cores"] >= 1 and o["value"] > 0
    assert o["static"]["value"] > 0 and o["dynamic64"]["value"] > 0
    assert o["env"]["OMP_PROC_BIND"] == "close"
