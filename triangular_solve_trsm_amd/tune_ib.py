"""Offline block-size profiling for the blocked path; writes csrc/ib_table.inc.

The adaptive blocking of HSMA-TRSM ("Hierarchical Shared Memory-Aware
Optimization for TRSM on GPU Platforms", section 4.3.2, Figure 8) has two
phases: offline, every candidate block size is timed for each (matrix scale,
data type) and only the fastest is kept in a table; online, the library looks
up the entry of the nearest tabulated scale.  This script is the offline
phase for MI355X; the online lookup is trsm_lln_select_ib in the library.
Besides the block size, each point times both orders of phase 2 (left-looking
as in section 4.3 "Phase 2", and right-looking) and the table keeps the
faster pair.

Protocol (section 5.1 of the pages): inputs drawn by trsm_inputs, each point
run 10 times, the first discarded, the mean of the last 9 kept.  B is
restored from a pristine copy before every run, outside the timed region.
Problems: square (m = n, the pages' scales) and, for each m, narrow ones
with n = 64, 256 and 1024 (below m), because a narrow B changes the balance
between the fixed costs of a block size and the GEMM work; the library looks
up the nearest (m, n).

Usage (on an MI355X, library built):
    python triangular_solve_trsm_amd/tune_ib.py [--sizes 128,256,...] [--out PATH]
then rebuild the library so that the new table is compiled in.
"""
from __future__ import annotations

import argparse
import datetime
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CANDIDATES = (64, 128, 256, 512, 1024)
DTYPES = (("f32", "R32F"), ("f64", "R64F"), ("c64", "C64F"), ("c32", "C32F"))
DEFAULT_SIZES = (128, 256, 512, 1024, 2048, 4096, 8192, 16384)
NARROW_N = (64, 256, 1024)


SCHEDULES = ("right", "left")


def time_point(T, torch, Ad, B0, alpha, ib, schedule, runs=10):
    os.environ["TRSM_SCHEDULE"] = schedule
    Bd = B0.clone()
    times = []
    for _ in range(runs):
        Bd.copy_(B0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        T.trsm_lln_ex(Ad, Bd, alpha, ib=ib, force_blocked=True)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del Bd
    return sum(times[1:]) / (runs - 1)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--sizes", default=",".join(str(s) for s in DEFAULT_SIZES))
    ap.add_argument("--out", default=os.path.join(HERE, "csrc", "ib_table.inc"))
    ap.add_argument("--json", default=None, help="also write every timing to this file")
    args = ap.parse_args()
    sizes = [int(s) for s in args.sizes.split(",") if s]

    import torch
    import triangular_solve_trsm_amd as T
    from trsm_inputs import make_problem

    assert torch.cuda.is_available(), "the sweep runs on the GPU"
    props = torch.cuda.get_device_properties(0)
    device = f"{getattr(props, 'gcnArchName', props.name)} ({props.multi_processor_count} CUs)"
    results = []
    best = {}
    import numpy as np
    for dt, code in DTYPES:
        for m in sizes:
            # one L and one square B per order; the narrow problems use the
            # first n columns of that B
            L, B = make_problem(dt, m, m, seed=20261300 + m)
            Ad = torch.from_numpy(np.ascontiguousarray(L.T)).cuda().T
            Bsq = torch.from_numpy(np.ascontiguousarray(B.T)).cuda().T
            del L, B
            alpha = 1.0 + 0j if dt in ("c64", "c32") else 1.0
            for n in [w for w in NARROW_N if w < m] + [m]:
                B0 = Bsq[:, :n]
                row = {}
                for ib in CANDIDATES:
                    if ib > m:
                        continue
                    for sch in SCHEDULES:
                        ms = time_point(T, torch, Ad, B0, alpha, ib, sch)
                        row[(ib, sch)] = ms
                        results.append({"dtype": dt, "m": m, "n": n, "ib": ib, "schedule": sch, "ms": ms})
                        print(json.dumps(results[-1]), flush=True)
                best[(code, m, n)] = (min(row, key=row.get), row)
            del Ad, Bsq
            torch.cuda.empty_cache()
    os.environ.pop("TRSM_SCHEDULE", None)

    stamp = datetime.date.today().isoformat()
    lines = [
        "// Diagonal block size by (data type, m, n), used with a nearest-scale",
        "// match (section 4.3.2 of the pages: offline profiling, online lookup).",
        "// Written by triangular_solve_trsm_amd/tune_ib.py on",
        f"// {device}, {stamp}: mean of runs 2-10 per point.",
        "// Fields: data type, order m, columns n, block size, phase-2 order",
        "// (1 left-looking, 0 right-looking).  Each entry's comment lists the time",
        "// in ms of every candidate block size, right-looking / left-looking.",
        "static const IbEntry kIbTable[] = {",
    ]
    for (code, m, n), ((ib, sch), row) in best.items():
        ibs = sorted({c for c, _ in row})
        times = ", ".join(f"{c}: {row[(c, 'right')]:.3f}/{row[(c, 'left')]:.3f}" for c in ibs)
        lines.append(f"    {{{code}, {m}, {n}, {ib}, {1 if sch == 'left' else 0}}},  // {times}")
    lines.append("};")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {args.out}", flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(results, f, indent=1)


if __name__ == "__main__":
    main()
