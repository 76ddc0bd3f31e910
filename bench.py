"""SpMV benchmark on one MI355X: y <- A*x + y, fp32, synthetic matrices.

Headline: the power-law matrix (4,000,000 rows, Zipf-like row lengths, about
65M nonzeros), the largest workload, in the format the automatic build picks.
One step = one full y <- A x + y pass with every input resident in HBM and
the caches flushed just before it (a 1 GiB fill kernel, untimed), timed with
HIP events on the stream the kernels run on.  The same line carries one entry
per other workload (2-D Laplacian 256^2, random 1M x 5, 27-point 128^3,
skewed 2M rows -- the last also in HYB with ELL width 20), every format's
figures on the headline matrix, the device's gather and LDS-update rates
(microbenchmarks), the builders' times and the CPU baselines.

GFLOP/s count 2 flops per nonzero; effective GB/s use the algorithmic bytes
    B_alg = 8*nnz + 4*(R+1) + 4*C + 8*R      (values+columns, row structure,
                                               x once, y read+write)
and the fraction is B_alg / time / 8 TB/s.  Before it is timed, every format's
y is checked row by row against an fp64 host product (scipy.sparse) within
1e-5 * (sum_j |a_ij x_j| + |y_i|); the oracle itself runs only in the
CPU-baseline leg.

    python bench.py [--steps K] [--warmup W] [--config cN] [--no-cpu]
"""
from __future__ import annotations

import os

# CPUs this process may use, recorded before an OpenMP runtime with thread
# binding pins the main thread to one of them
_AFFINITY_CPUS = len(os.sched_getaffinity(0))
# CPU baseline thread placement (read when the OpenMP runtime starts)
os.environ.setdefault("OMP_PROC_BIND", "close")
os.environ.setdefault("OMP_PLACES", "cores")

import argparse  # noqa: E402
import json  # noqa: E402
import statistics  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, vendor figure
FLUSH_BYTES = 1 << 30       # > 256 MB MALL + 8 x 4 MB L2
FORMATS = ["coo_atomic", "coo_segmented", "csr_scalar", "csr_vector", "ell", "hyb", "jds",
           "csr_merge", "sell", "ell_xtile", "coo_blocked"]
HEADLINE = "c5"
WORKLOAD_NAMES = {
    "c1": "laplacian2d_256 (65,536 rows, 5-point, 326,656 nnz)",
    "c2": "random_rows_1Mx5 (1,000,000 x 1,000,000, 5 random cols/row, 5,000,000 nnz)",
    "c3": "stencil27_128 (2,097,152 rows, 27-point truncated, 55,742,968 nnz)",
    "c4": "skewed_2M (2,000,000 rows, 10-20 nnz + 50 rows of 1000-5000)",
    "c5": "power_law_4M (4,000,000 rows, Zipf 2.1 row lengths, ~65M nnz)",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alg_bytes(R, C, nnz):
    return 8 * nnz + 4 * (R + 1) + 4 * C + 8 * R


def pages_bytes(R, nnz):
    """The pages' own traffic model: 12 B per nonzero (value, column and the x
    element it gathers) plus 8 B per row (y).  x elements are counted once per
    nonzero, so on cached x this is not a fraction of any peak."""
    return 12 * nnz + 8 * R


def input_hashes(w):
    import hashlib
    return {k: hashlib.sha256(getattr(w, k).tobytes()).hexdigest()[:16]
            for k in ("row_ptrs", "col_idx", "values", "x", "y")}


def copy_reference(torch, dev, flush_buf, steps=10):
    """A plain 512 MiB device-to-device copy by torch's elementwise kernel
    (dst = src + 0; 5.5 TB/s against 4.7 for the runtime's copy_ blit),
    timed like a step: what this device's HBM delivers to a simple streaming
    kernel, for context beside the 8 TB/s specification."""
    n = 512 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(steps):
        flush_buf.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        torch.add(src, 0.0, out=dst)
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    us = statistics.median(ts) * 1e3
    del src, dst
    gbs = 2 * n / (us * 1e-6) / 1e9
    return {"kernel": "device copy (torch elementwise dst = src + 0), 512 MiB read + "
                      "512 MiB written",
            "us_median": round(us, 2), "gbs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def time_format(spmv, torch, h, x, y, steps, warmup, flush_buf, flush=True):
    """Per-step kernel time (ms) with an untimed cache flush before each step."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        if flush:
            flush_buf.zero_()
        h.run(x, y)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        if flush:
            flush_buf.zero_()
        a.record(stream)
        h.run(x, y)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in evs], wall


def host_reference(w):
    """y_ref = A x + y in fp64 on the host (scipy.sparse, a library product
    independent of both the oracle and the HIP path) and the per-row bound
    1e-5 * (|A| |x| + |y|)."""
    import numpy as np
    import scipy.sparse as sp
    shape = (w.num_rows, w.num_cols)
    a = sp.csr_matrix((w.values.astype(np.float64), w.col_idx, w.row_ptrs), shape=shape)
    x = w.x.astype(np.float64)
    y = w.y.astype(np.float64)
    y_ref = a @ x + y
    a.data = np.abs(a.data)
    bound = 1e-5 * (a @ np.abs(x) + np.abs(y))
    return y_ref, bound


def check_rows(y, y_ref, bound):
    """(rows out of bound, first such row or -1, worst |error| / bound)."""
    import numpy as np
    err = np.abs(y.astype(np.float64) - y_ref)
    bad = np.nonzero(err > bound)[0]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return int(bad.size), int(bad[0]) if bad.size else -1, worst


def cpu_baseline(w, y_ref, bound, budget_s=10.0):
    """The oracle as it is (single thread, fp64 sums) on full passes of the
    same matrix, for about `budget_s` seconds (at least 3 passes; median), and
    beside it the OpenMP CSR baseline."""
    import oracle
    oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)  # load / warm
    ts, t_total = [], 0.0
    while t_total < budget_s or len(ts) < 3:
        t0 = time.perf_counter()
        oracle.spmv_csr(w.row_ptrs, w.col_idx, w.values, w.x, w.y)
        ts.append(time.perf_counter() - t0)
        t_total += ts[-1]
    t = statistics.median(ts)
    return {"value": round(2 * w.nnz / t / 1e9, 4), "unit": "GFLOP/s", "cores": 1,
            "kind": "oracle", "host": host_cpu(),
            "sample": f"{len(ts)} full passes of the same {w.num_rows}-row matrix "
                      f"({w.nnz} nnz), median {t * 1e3:.1f} ms, single thread, fp64 sums",
            "gbs_alg": round(alg_bytes(w.num_rows, w.num_cols, w.nnz) / t / 1e9, 3),
            "openmp": openmp_baseline(w, y_ref, bound)}


def host_cpu():
    """Model name and logical CPU count of the host the baseline ran on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count(), "affinity_cpus": _AFFINITY_CPUS}


def openmp_baseline(w, y_ref, bound, reps=10):
    """OpenMP CSR SpMV (oracle/csr_omp.c): rows over all OpenMP threads, fp32
    row sums, first-touch copies of the arrays, OMP_PROC_BIND=close; the
    median of `reps` timed passes with schedule(static) and with
    schedule(dynamic,64).  Each y is first checked against the oracle within
    the bound of recursive fp32 summation, (n + 2) * 2^-24 * (|y| + sum |a x|)."""
    import numpy as np
    import oracle
    out = {"kind": "openmp_csr", "unit": "GFLOP/s", "cores": oracle.omp_threads(),
           "env": {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OMP_PROC_BIND",
                                                  "OMP_PLACES")}}
    n = np.diff(w.row_ptrs.astype(np.int64))
    mag = bound / 1e-5
    B = alg_bytes(w.num_rows, w.num_cols, w.nnz)
    for label, dyn in (("static", False), ("dynamic64", True)):
        y, t = oracle.spmv_csr_omp(w.row_ptrs, w.col_idx, w.values, w.x, w.y, dynamic=dyn,
                                   reps=reps)
        err = np.abs(y.astype(np.float64) - y_ref)
        bad = int(np.sum(err > (n + 2) * 2.0**-24 * mag))
        if bad:
            raise RuntimeError(f"OpenMP CSR baseline ({label}): {bad} rows out of bound")
        out[label] = {"value": round(2 * w.nnz / t / 1e9, 3), "ms_median": round(t * 1e3, 3),
                      "gbs_alg": round(B / t / 1e9, 2)}
    best = max(("static", "dynamic64"), key=lambda k: out[k]["value"])
    out["value"] = out[best]["value"]
    out["schedule"] = best
    out["sample"] = (f"median of {reps} full passes per schedule of the same "
                     f"{w.num_rows}-row matrix, {out['cores']} OpenMP threads, fp32 row sums")
    return out


def run_config(spmv, torch, dev, cfg, steps, warmup, flush_buf, formats=False, fmt="auto",
               col_blocks=0, log_prefix=""):
    """Build and time one workload.  Returns (entry, context) where entry is the
    JSON-ready summary of the selected format (and, if asked, every format) and
    context keeps what the headline needs (handle, tensors, times)."""
    from spmv_storage_formats_amd import synth
    log(f"{log_prefix}generating {cfg}")
    w = synth.workload(cfg)
    R, C, nnz = w.num_rows, w.num_cols, w.nnz
    B = alg_bytes(R, C, nnz)
    flops = 2 * nnz
    rp = torch.from_numpy(w.row_ptrs).to(dev)
    ci = torch.from_numpy(w.col_idx).to(dev)
    va = torch.from_numpy(w.values).to(dev)
    x = torch.from_numpy(w.x).to(dev)
    y0 = torch.from_numpy(w.y).to(dev)
    y_ref, bound = host_reference(w)

    def build_and_check(f, **kw):
        if col_blocks:
            kw.setdefault("col_blocks", col_blocks)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h = spmv.build(f, rp, ci, va, C, **kw)
        bms = (time.perf_counter() - t0) * 1e3
        y = y0.clone()
        h.run(x, y)
        torch.cuda.synchronize()
        n_bad, first, worst = check_rows(y.cpu().numpy(), y_ref, bound)
        if n_bad:
            raise SystemExit(f"parity failure {cfg}/{f}: {n_bad} rows (first {first})")
        return h, bms, worst

    def summary(h, times, bms, worst):
        med = statistics.median(times)
        mean = statistics.mean(times)
        prof = profiled_entry(f"{cfg}/{h.format}")
        traffic = prof["hbm_bytes_per_launch"] if prof else None
        prof_us = prof.get("kernel_avg_us") if prof else None
        e = {"format": h.format, "col_blocks": h.info["col_blocks"],
             "us_median": round(med * 1e3, 2), "us_mean": round(mean * 1e3, 2),
             "gflops": round(flops / (mean * 1e-3) / 1e9, 1),
             "gbs_alg": round(B / (mean * 1e-3) / 1e9, 1),
             "frac_by_events": round(B / (mean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "profiled_kernel": prof.get("kernel") if prof else None,
             "profiled_kernel_us": prof_us,
             "frac_by_profiled_kernel_us": (round(B / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                            if prof_us else None),
             "traffic_bytes": traffic,
             "traffic_over_alg": round(traffic / B, 3) if traffic else None,
             "frac_by_counter_bytes": (round(traffic / (prof_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                       if traffic and prof_us else None),
             "build_ms": round(bms, 2), "device_MB": round(h.info["device_bytes"] / 1e6, 1),
             "worst_err_over_bound": float(f"{worst:.3g}")}
        return e

    per_format = {}
    if formats:
        for f in FORMATS:
            try:
                hf, bms, wst = build_and_check(f, **({"hyb_width": 20} if cfg == "c4" else {}))
            except spmv.SpmvError as e:
                per_format[f] = {"refused": e.name}
                continue
            tf, _ = time_format(spmv, torch, hf, x, y0.clone(), max(10, steps // 2), 2,
                                flush_buf)
            per_format[f] = summary(hf, tf, bms, wst)
            log(f"{log_prefix}{cfg} {f}: {per_format[f]['us_median']} us")
            hf.close()
    log(f"{log_prefix}{cfg}: building {fmt}")
    h, bms, worst = build_and_check(fmt)
    y = y0.clone()
    times, wall = time_format(spmv, torch, h, x, y, steps, warmup, flush_buf)
    entry = {"workload": WORKLOAD_NAMES[cfg], "rows": R, "cols": C, "nnz": nnz,
             "alg_bytes": B, **summary(h, times, bms, worst)}
    log(f"{log_prefix}{cfg}: {entry['format']} {entry['us_median']} us, "
        f"frac {entry['frac_by_events']}")
    if cfg == "c4":
        # the configuration names HYB with ELL width 20: reported beside the
        # automatic format
        hh, hbms, hw = build_and_check("hyb", hyb_width=20)
        th, _ = time_format(spmv, torch, hh, x, y0.clone(), max(10, steps // 2), 2, flush_buf)
        entry["hyb_width20"] = summary(hh, th, hbms, hw)
        hh.close()
    if per_format:
        entry["formats"] = per_format
    ctx = {"w": w, "h": h, "times": times, "wall": wall, "x": x, "y0": y0, "y_ref": y_ref,
           "bound": bound, "B": B}
    return entry, ctx


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None, choices=sorted(WORKLOAD_NAMES),
                    help="time only this workload (as the headline); default: the power-law "
                         "matrix as the headline plus one entry per other workload")
    ap.add_argument("--format", default="auto")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only-selected", action="store_true",
                    help="time only the selected format of the headline workload (for "
                         "profiling runs)")
    ap.add_argument("--all-formats", action="store_true",
                    help="every format on every workload (default: on the headline only)")
    ap.add_argument("--no-micro", action="store_true", help="skip the microbenchmarks")
    ap.add_argument("--warm", action="store_true",
                    help="also time the selected format without cache flushes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--col-blocks", type=int, default=0,
                    help="x slices for every build (0 = library default)")
    ap.add_argument("--cg", action="store_true",
                    help="also run conjugate gradient on the 256^2 and 2048^2 Laplacians "
                         "and report the per-iteration cost")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy 5 times (reads 512 MiB, writes "
                         "512 MiB per launch) to scale PMC byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this engine runs on one GPU; --gpus N > 1 is not supported "
              "(the row-sharded multi-GPU design is documented, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import spmv_storage_formats_amd as spmv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    spmv.load_library()
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    headline = args.config or HEADLINE
    others = [] if (args.config or args.only_selected) else \
        [c for c in ("c1", "c2", "c3", "c4") if c != headline]

    configs = {}
    for cfg in others:
        entry, ctx = run_config(spmv, torch, dev, cfg, min(args.steps, 30), args.warmup,
                                flush_buf, formats=args.all_formats, col_blocks=args.col_blocks)
        ctx["h"].close()
        configs[cfg] = entry
        del ctx
        torch.cuda.empty_cache()

    entry, ctx = run_config(spmv, torch, dev, headline, args.steps, args.warmup, flush_buf,
                            formats=not args.only_selected, fmt=args.format,
                            col_blocks=args.col_blocks)
    configs[headline] = entry
    w, h, times, wall, B = ctx["w"], ctx["h"], ctx["times"], ctx["wall"], ctx["B"]
    R, C, nnz = w.num_rows, w.num_cols, w.nnz
    flops = 2 * nnz
    ms = statistics.mean(times)
    med = statistics.median(times)
    gbs = B / (ms * 1e-3) / 1e9
    warm_ms = warm_med = None
    if args.warm:
        warm_times, _ = time_format(spmv, torch, h, ctx["x"], ctx["y0"].clone(), args.steps,
                                    args.warmup, flush_buf, flush=False)
        warm_ms = round(statistics.mean(warm_times), 5)
        warm_med = round(statistics.median(warm_times), 5)
    q = statistics.quantiles(times, n=10) if len(times) >= 2 else [med] * 9
    prof = profiled_entry(f"{headline}/{h.format}")
    traffic = prof["hbm_bytes_per_launch"] if prof else None
    prof_us = prof.get("kernel_avg_us") if prof else None
    l2_req = prof.get("l2_requests_per_launch") if prof else None
    overhead_us = event_overhead_us(torch)

    result = {
        "metric": "SpMV GFLOP/s and effective HBM GB/s (% of MI355X peak) per format, 1 GPU",
        "value": round(flops / (ms * 1e-3) / 1e9, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded), inputs resident in HBM, caches flushed before each step",
        "config": {"workload": WORKLOAD_NAMES[headline], "format": h.format,
                   "col_blocks": h.info["col_blocks"],
                   "rows": R, "cols": C, "nnz": nnz, "max_row_length": int(h.info["max_len"]),
                   "parallelism": "single GPU", "inputs_sha256": input_hashes(w)},
        "effective_gbs": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "ms_median": round(med, 5),
        "event_overhead_us": overhead_us,
        "step_us": {"p10": round(q[0] * 1e3, 2), "median": round(med * 1e3, 2),
                    "p90": round(q[8] * 1e3, 2), "mean": round(ms * 1e3, 2)},
        "warm_ms_per_step": warm_ms,
        "warm_ms_median": warm_med,
        "pages_model_gbs": round(pages_bytes(R, nnz) / (ms * 1e-3) / 1e9, 1),
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "build_ms": entry["build_ms"],
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch_alg": B,
                     "kernel": prof.get("kernel") if prof else None,
                     # the same kernel's average duration in the committed
                     # rocprofv3 trace of this workload (no dispatch latency)
                     # and the fractions it gives, beside the live event time
                     "profiled_kernel_us": prof_us,
                     "frac_by_profiled_kernel_us": (round(B / (prof_us * 1e-6) / 1e9 /
                                                          HBM_PEAK_GBS, 4)
                                                    if prof_us else None),
                     "traffic_over_alg": round(traffic / B, 3) if traffic else None,
                     "l2_requests_per_launch": l2_req,
                     "l2_g_requests_per_s_by_profiled_kernel_us": (
                         round(l2_req / (prof_us * 1e-6) / 1e9, 1)
                         if l2_req and prof_us else None),
                     "spmv_g_gathers_per_s": round(nnz / (med * 1e3) / 1e3, 1)},
        "configs": configs,
    }
    if not args.no_micro:
        from spmv_storage_formats_amd import microbench
        log("microbenchmarks")
        result["device_rates"] = {"gather": microbench.gather_rates(torch, dev, flush_buf),
                                  "lds": microbench.lds_rates(torch, dev)}
    cref = copy_reference(torch, dev, flush_buf)
    cref["spmv_frac_of_copy"] = round(gbs / cref["gbs"], 4)
    result["copy_reference"] = cref
    if not args.only_selected:
        result["coo_to_csr"] = coo_section(spmv, torch, w, dev)
    if args.cg:
        from spmv_storage_formats_amd import synth
        result["cg"] = cg_section(spmv, torch, synth, dev, flush_buf)
    if args.calibrate_copy:
        n = 512 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            flush_buf.zero_()
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = {"read": n, "write": n}
    if not args.no_cpu:
        log("cpu baseline (oracle, OpenMP)")
        result["cpu_baseline"] = cpu_baseline(w, ctx["y_ref"], ctx["bound"], args.cpu_seconds)
    print(json.dumps(result), flush=True)


def coo_section(spmv, torch, w, dev):
    """COO -> CSR on the device for the same matrix given as a COO list in
    random order (the stable-sort path) and in row order (count and scan
    only): median of 5 host-timed calls, each host-synchronous."""
    import numpy as np
    rows = np.repeat(np.arange(w.num_rows, dtype=np.int32), np.diff(w.row_ptrs))
    p = np.random.default_rng(0).permutation(w.nnz)
    out = {}
    for label, order in (("shuffled", p), ("row_sorted", None)):
        sel = (lambda a: a[order]) if order is not None else (lambda a: a)
        ri = torch.from_numpy(sel(rows)).to(dev)
        ci = torch.from_numpy(sel(w.col_idx)).to(dev)
        va = torch.from_numpy(sel(w.values)).to(dev)
        spmv.coo_to_csr(ri, ci, va, w.num_rows, w.num_cols)
        ts = []
        for _ in range(5):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            spmv.coo_to_csr(ri, ci, va, w.num_rows, w.num_cols)
            ts.append(time.perf_counter() - t0)
        ms = statistics.median(ts) * 1e3
        out[label + "_ms"] = round(ms, 3)
        out[label + "_g_entries_per_s"] = round(w.nnz / ms / 1e6, 2)
        del ri, ci, va
    return out


def cg_section(spmv, torch, synth, dev, flush_buf):
    """Conjugate gradient on 2-D Laplacians: iterations, time per iteration and
    the share of it spent in SpMV (the step the pages call the core of the
    method).  The 256^2 grid is solved to rtol 1e-5 from b = A x_true; the
    2048^2 grid (4.2M rows) runs a fixed 200 iterations to time the
    bandwidth-bound regime."""
    import numpy as np
    import scipy.sparse as sp
    out = []
    for n, fixed in ((256, 0), (2048, 200)):
        w = synth.laplacian2d(n)
        a = sp.csr_matrix((w.values.astype(np.float64), w.col_idx, w.row_ptrs),
                          shape=(w.num_rows, w.num_cols))
        b = a @ w.x.astype(np.float64)
        bt = torch.from_numpy(b.astype(np.float32)).to(dev)
        h = spmv.build("auto", torch.from_numpy(w.row_ptrs).to(dev),
                       torch.from_numpy(w.col_idx).to(dev), torch.from_numpy(w.values).to(dev),
                       w.num_cols)
        xg = torch.zeros(w.num_rows, device=dev)
        h.cg(bt, xg, max_iter=16, rtol=0.0)             # warm-up
        xg.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if fixed:
            iters, rel = h.cg(bt, xg, max_iter=fixed, rtol=0.0)
        else:
            iters, rel = h.cg(bt, xg, max_iter=5000, rtol=1e-5)
        torch.cuda.synchronize()
        total = time.perf_counter() - t0
        xs, ys = torch.ones(w.num_rows, device=dev), torch.zeros(w.num_rows, device=dev)
        tf, _ = time_format(spmv, torch, h, xs, ys, 50, 5, flush_buf, flush=False)
        spmv_ms = statistics.median(tf)
        per_it = total * 1e3 / max(iters, 1)
        # algorithmic bytes per iteration: the SpMV's plus 48 B per row of vector
        # traffic (p.Ap reads 8; the x, r update reads 16 and writes 8; the new
        # direction reads 8 and writes 8)
        it_bytes = alg_bytes(w.num_rows, w.num_cols, w.nnz) + 48 * w.num_rows
        entry = {"workload": f"laplacian2d_{n} ({w.num_rows:,} rows, {w.nnz:,} nnz), "
                             f"b = A x_true, x0 = 0, "
                             + (f"{fixed} iterations" if fixed else "rtol 1e-5"),
                 "format": h.format, "iterations": iters, "rel_residual": rel,
                 "total_ms": round(total * 1e3, 3), "ms_per_iteration": round(per_it, 5),
                 "spmv_ms_warm": round(spmv_ms, 5),
                 "spmv_share": round(spmv_ms / per_it, 3),
                 "alg_bytes_per_iteration": it_bytes,
                 "gbs_per_iteration": round(it_bytes / (per_it * 1e-3) / 1e9, 1)}
        if not fixed:
            entry["max_abs_error"] = float(np.max(np.abs(xg.cpu().numpy() - w.x)))
        out.append(entry)
        h.close()
    return out


def event_overhead_us(torch):
    """Median HIP-event time around one empty kernel (torch's spin kernel with
    a zero count) on the same stream: the dispatch latency that per-step event
    timing adds to a kernel's execution time (rocprofv3 counts execution only)."""
    stream = torch.cuda.current_stream()
    times = []
    for i in range(60):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        torch.cuda._sleep(0)
        b.record(stream)
        b.synchronize()
        if i >= 10:
            times.append(a.elapsed_time(b))
    return round(statistics.median(times) * 1e3, 2)


def profiled_entry(key):
    """The committed PMC summary entry for `key` (profiles/*_pmc_traffic.md, a
    JSON block each): HBM bytes per launch and the kernel's average duration
    in the matching rocprofv3 kernel trace.  None when no summary has the key
    or the kernels changed since it was taken."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    table = {}
    for f in sorted(os.listdir(pdir)):
        if not f.endswith("_pmc_traffic.md"):
            continue
        text = open(os.path.join(pdir, f)).read()
        start = text.find("```json")
        if start < 0:
            continue
        end = text.find("```", start + 7)
        table.update(json.loads(text[start + 7:end]))
    entry = table.get(key)
    if entry and entry.get("kernel_source_sha") == kernel_source_sha():
        return entry
    return None


def measured_traffic(key):
    """HBM bytes per launch from the committed PMC summaries, or None."""
    entry = profiled_entry(key)
    return entry["hbm_bytes_per_launch"] if entry else None


def kernel_source_sha():
    """Hash of the code the SpMV kernels are compiled from (the kernels files
    and the shared header; the blocked-COO builder shares its file), with
    comments and whitespace removed, so that an edit to a comment keeps the
    profiles valid and any change to the code does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "spmv_storage_formats_amd", "csrc")
    for f in ("internal.h", "spmv_kernels.hip", "coo_blocked.hip"):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
