"""Time the library on every workload it is measured on, one JSON line each.

bench.py times the headline step (fp64 8192^2 solve plus the batched complex
64 x 64 solve); this script times each workload on its own:

  * the five configurations (fp64 64^2; batched complex 64^2 x 8192; fp32
    4096^2 with alpha 0.5; fp64 8192^2; complex 8192 x 2048);
  * narrow right-hand sides (m = 8192, n = 64 / 256), where the phase-2
    products split along K;
  * complex fp32 at the fp32 and complex configurations' shapes;
  * general TRSM variants (right side, upper triangle, transposes, unit
    diagonal) at fp64 4096^2, against trsm_lln on the same data.

Protocol: inputs from trsm_inputs (seeded), moved to the GPU; a sustained
warm-up of about 0.3 s of the same call (the GPU clock drops while the host
prepares inputs); then 30 timed calls, B restored from a pristine copy
outside the events; the median is reported.  Rates count m^2 n flops (4 m^2 n
complex); fractions are of MI355X's fp32 (157.3 TFLOP/s) or fp64
(78.6 TFLOP/s) matrix peak, and of 8 TB/s HBM for the batched solve.

Usage (on an MI355X, library built):
    python triangular_solve_trsm_amd/bench_workloads.py [--only SUBSTR,...]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"f32": 157.3e12, "c32": 157.3e12, "f64": 78.6e12, "c64": 78.6e12}
ESIZE = {"f32": 4, "c32": 8, "f64": 8, "c64": 16}
HBM = 8.0e12


def to_dev(torch, np, a):
    if a.ndim == 2:
        return torch.from_numpy(np.ascontiguousarray(a.T)).cuda().T
    return torch.from_numpy(np.ascontiguousarray(np.transpose(a, (0, 2, 1)))).cuda().transpose(1, 2)


def timed_median(torch, call, restore, runs=30, warm_s=0.3):
    t0 = time.time()
    while time.time() - t0 < warm_s:
        restore()
        call()
    torch.cuda.synchronize()
    ts = []
    for _ in range(runs):
        restore()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return statistics.median(ts), min(ts)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--only", default="", help="comma-separated substrings of workload names")
    args = ap.parse_args()
    only = [s for s in args.only.split(",") if s]

    import numpy as np
    import torch

    import triangular_solve_trsm_amd as T
    from trsm_inputs import CONFIGS, make_config, make_problem

    assert torch.cuda.is_available(), "the workloads run on the GPU"
    codes = {"f32": T.R32F, "f64": T.R64F, "c64": T.C64F, "c32": T.C32F}

    def wanted(name):
        return not only or any(o in name for o in only)

    def report(name, dt, m, n, batch, med, mn, extra=None):
        fl = (4.0 if dt in ("c64", "c32") else 1.0) * m * m * n * batch
        rec = {"workload": name, "dtype": dt, "m": m, "n": n, "batch": batch, "median_ms": round(med, 4),
               "min_ms": round(mn, 4), "tflops": round(fl / (med * 1e-3) / 1e12, 2),
               "frac_peak": round(fl / (med * 1e-3) / PEAK[dt], 4)}
        if batch > 1:
            byts = ESIZE[dt] * (m * (m + 1) // 2 + 2 * m * n) * batch
            rec["frac_hbm"] = round(byts / (med * 1e-3) / HBM, 4)
        elif m > 64:
            rec["ib"] = T.trsm_lln_select_ib(codes[dt], m, n)
        if extra:
            rec.update(extra)
        print(json.dumps(rec), flush=True)

    # the five configurations
    for name, cfg in CONFIGS.items():
        if not wanted(name):
            continue
        L, B, a = make_config(cfg)
        Ad, B0 = to_dev(torch, np, L), to_dev(torch, np, B)
        Bd = B0.clone()
        del L, B
        if cfg.batch:
            call = lambda: T.trsm_lln_strided_batched(Ad, Bd, a)  # noqa: E731
        else:
            call = lambda: T.trsm_lln(Ad, Bd, a)  # noqa: E731
        med, mn = timed_median(torch, call, lambda: Bd.copy_(B0))
        report(name, cfg.dtype, cfg.m, cfg.n, cfg.batch or 1, med, mn)
        del Ad, B0, Bd
        torch.cuda.empty_cache()

    # narrow right-hand sides and complex fp32
    extra_shapes = [("narrow_f64_8192x64", "f64", 8192, 64), ("narrow_f64_8192x256", "f64", 8192, 256),
                    ("narrow_c64_8192x64", "c64", 8192, 64), ("narrow_c64_8192x256", "c64", 8192, 256),
                    ("narrow_f32_8192x64", "f32", 8192, 64), ("c32_4096x4096", "c32", 4096, 4096),
                    ("c32_8192x2048", "c32", 8192, 2048)]
    for name, dt, m, n in extra_shapes:
        if not wanted(name):
            continue
        L, B = make_problem(dt, m, n, seed=m + n)
        Ad, B0 = to_dev(torch, np, L), to_dev(torch, np, B)
        Bd = B0.clone()
        del L, B
        a = 1.0 + 0j if dt in ("c64", "c32") else 1.0
        med, mn = timed_median(torch, lambda: T.trsm_lln(Ad, Bd, a), lambda: Bd.copy_(B0))
        report(name, dt, m, n, 1, med, mn)
        del Ad, B0, Bd
        torch.cuda.empty_cache()

    # general TRSM variants against the left-lower solve on the same data
    variants = [("L", "L", "N", "U"), ("L", "U", "N", "N"), ("L", "U", "T", "N"), ("L", "L", "C", "N"),
                ("R", "L", "N", "N"), ("R", "U", "T", "N")]
    if any(wanted(f"variant_f64_4096_{''.join(v)}") for v in variants):
        m = n = 4096
        L, B = make_problem("f64", m, n, seed=4096)
        # a matrix whose both triangles are well conditioned: L plus L^T
        # minus the diagonal, so every variant solves a lower or upper
        # triangle of the same values
        F = L + L.T - np.diag(np.diag(L))
        Ad, B0 = to_dev(torch, np, np.asfortranarray(F)), to_dev(torch, np, B)
        Bd = B0.clone()
        del L, B, F
        base, _ = timed_median(torch, lambda: T.trsm_lln(Ad, Bd, 1.0), lambda: Bd.copy_(B0))
        for side, uplo, trans, diag in variants:
            name = f"variant_f64_4096_{side}{uplo}{trans}{diag}"
            if not wanted(name):
                continue
            med, mn = timed_median(
                torch, lambda: T.trsm_solve(Ad, Bd, 1.0, side=side, uplo=uplo, trans=trans, diag=diag),
                lambda: Bd.copy_(B0))
            report(name, "f64", m, n, 1, med, mn, {"vs_trsm_lln": round(med / base, 4)})
        del Ad, B0, Bd
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
