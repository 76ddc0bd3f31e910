"""Gather and LDS-update rates of the device, measured by the microbenchmark
kernels of ``bench_csrc/microbench.hip`` (benchmark support, not the SpMV
library).

    python -m spmv_storage_formats_amd.microbench      # one JSON line

``gather_rates``: 64M 4-byte gathers x[idx[i]] per pattern, each timed with
HIP events after a 1 GiB cache flush (median of 9): random indices, indices
sorted inside each 64-lane group with mean spacing 16, 8 or 4 (two, four or
eight lanes per 128-byte line), the four-per-line sets with each group's
lanes shuffled, and consecutive indices; from an x of 2 MiB (one
XCD's L2 keeps it with room to spare), 4 MiB (the size of an L2), 8 MiB and
16 MiB.
``lds_rates``: random-address float adds into LDS, 512 workgroups of 1024
threads x 2048 adds each, by the hardware float atomic, a compare-and-swap
loop and the integer atomic; reported as GPU clocks per wave instruction per
CU (2.4 GHz, 256 CUs).
"""
from __future__ import annotations

import ctypes
import json
import os
import statistics
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_PKG, "libspmv_microbench.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            from . import _build
            _build.build_microbench()
        lib = ctypes.CDLL(_LIB)
        lib.mb_gather.restype = ctypes.c_int
        lib.mb_gather.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
        lib.mb_gather_out_len.restype = ctypes.c_int64
        lib.mb_gather_out_len.argtypes = [ctypes.c_int64]
        lib.mb_lds_update.restype = ctypes.c_int
        lib.mb_lds_update.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def _time(torch, fn, flush, reps=9):
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return statistics.median(ts) * 1e3   # us


def _patterns(torch, dev, n, X, gen):
    """Index tensors (int32) of n gathers from an x of X floats.  The
    shuffled pattern holds the same index sets per 64-lane group as the
    4-per-line one, each group's lanes in a random order."""
    g = n // 64
    out = {"random": torch.randint(0, X, (n,), device=dev, generator=gen, dtype=torch.int64)}
    start = torch.randint(0, X, (g, 1), device=dev, generator=gen, dtype=torch.int64)
    for name, hi in (("sorted_2_per_line", 32), ("sorted_4_per_line", 16),
                     ("sorted_8_per_line", 8)):
        gaps = torch.randint(1, hi, (g, 64), device=dev, generator=gen, dtype=torch.int64)
        idx = (start + torch.cumsum(gaps, dim=1)) % X
        out[name] = idx.reshape(-1)
        if hi == 16:
            perm = torch.argsort(torch.rand(g, 64, device=dev, generator=gen), dim=1)
            out["sorted_4_per_line_shuffled"] = torch.gather(idx, 1, perm).reshape(-1)
    out["consecutive"] = torch.arange(n, device=dev, dtype=torch.int64) % X
    return {k: v.to(torch.int32) for k, v in out.items()}


def gather_rates(torch, dev, flush, n=64 << 20):
    lib = _load()
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    out = torch.empty(int(lib.mb_gather_out_len(n)), device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for mib in (2, 4, 8, 16):
        X = (mib << 20) // 4
        x = torch.rand(X, device=dev, generator=gen)
        for name, idx in _patterns(torch, dev, n, X, gen).items():
            assert int(idx.min()) >= 0 and int(idx.max()) < X
            def fn():
                if lib.mb_gather(n, idx.data_ptr(), x.data_ptr(), out.data_ptr(), stream) != 0:
                    raise RuntimeError("mb_gather launch failed")
            us = _time(torch, fn, flush)
            res[f"x{mib}MiB_{name}"] = {"us": round(us, 1), "g_per_s": round(n / us / 1e3, 1)}
            del idx
    return {"gathers": n, "rates": res}


def lds_rates(torch, dev, blocks=512, iters=2048):
    lib = _load()
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    addr = torch.randint(0, 16384, (4096,), device=dev, generator=gen,
                         dtype=torch.int64).to(torch.int32)
    out = torch.empty(blocks * 1024, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for mode, name in ((0, "lds_float_atomic_add"), (1, "cas_float_add"),
                       (2, "lds_integer_atomic_add")):
        def fn():
            if lib.mb_lds_update(mode, blocks, iters, addr.data_ptr(), out.data_ptr(),
                                 stream) != 0:
                raise RuntimeError("mb_lds_update launch failed")
        us = _time(torch, fn, None, reps=5)
        wave_instr = blocks * 16 * iters
        res[name] = {"us": round(us, 1),
                     "clocks_per_wave_instruction": round(us * 1e-6 * 2.4e9 * 256 / wave_instr, 1)}
    return res


def main():
    import torch
    dev = torch.device("cuda:0")
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    print(json.dumps({"gather": gather_rates(torch, dev, flush), "lds": lds_rates(torch, dev)}),
          flush=True)


if __name__ == "__main__":
    sys.exit(main())
