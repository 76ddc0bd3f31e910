"""bench.py's one-line JSON result on the GPU: the fields and their relations
(the default 1M x 5 random workload, shortened timing and CPU baseline)."""
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
                        "--warmup", "1", "--only-selected", "--cpu-seconds", "0.5"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    out = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(out) == 1, p.stdout[-2000:]
    return json.loads(out[0])


def test_contract_fields(line):
    d = line
    assert d["metric"].startswith("SpMV GFLOP/s") and d["unit"] == "GFLOP/s"
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["dtype"] == "f32"
    assert d["data"].startswith("synthetic")
    cfg = d["config"]
    assert cfg["workload"].startswith("random_rows_1Mx5")
    assert (cfg["rows"], cfg["cols"], cfg["nnz"]) == (1_000_000, 1_000_000, 5_000_000)
    assert cfg["format"] == "ell"
    # value = 2 nnz / mean step time
    assert d["value"] > 0
    assert abs(d["value"] - 2 * cfg["nnz"] / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]


def test_roofline_fields(line):
    r = line["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    # algorithmic bytes: 8 per nonzero, row pointers, x once, y read and written
    R = C = 1_000_000
    nnz = 5_000_000
    assert r["bytes_per_launch_alg"] == 8 * nnz + 4 * (R + 1) + 4 * C + 8 * R
    assert abs(r["achieved"] - r["bytes_per_launch_alg"] / (line["ms_per_step"] * 1e-3) / 1e9) \
        <= 0.01 * r["achieved"]
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-3
    assert 0 < r["frac"] < 1
    # traffic and the profiled duration come from the committed summaries, or
    # are null when the kernel sources changed since they were taken
    assert r["traffic"] is None or (isinstance(r["traffic"], int) and r["traffic"] > 0)
    assert (r["profiled_kernel_us"] is None) == (r["traffic"] is None)
    # L2 requests from the same summaries: about one per random gather
    if r["l2_requests_per_launch"] is not None:
        assert r["l2_requests_per_launch"] >= nnz
        rate = r["l2_requests_per_launch"] / (line["ms_per_step"] * 1e-3) / 1e9
        assert abs(r["l2_g_requests_per_s"] - rate) <= 0.01 * rate


def test_cpu_baseline_fields(line):
    c = line["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "GFLOP/s" and c["cores"] == 1
    assert c["value"] > 0 and "full passes" in c["sample"]
    o = c["openmp"]
    assert o["kind"] == "openmp_csr" and o["cores"] >= 1 and o["value"] > 0
