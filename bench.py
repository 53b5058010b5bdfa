"""Benchmark of the MI355X left-lower TRSM library on its headline workloads.

One step = one pass of the whole hot path over one batch of synthetic input:
  * the fp64 solve L X = B with m = n = 8192 (blocked path: diagonal-block
    inversion, then per block row an MFMA solve GEMM and an MFMA trailing
    update GEMM), and
  * the batched complex-fp64 solve of 8192 independent 64 x 64 systems
    (direct single-workgroup kernel, HBM bound).
Both solves run in place, so step s solves with the X of step s-1 as its
right-hand side: every step is a complete TRSM of the same size.

Reported (one JSON line on stdout):
  value        whole-job GFLOP/s (counted flops m^2 n real, 4 m^2 n complex)
               over the K timed steps, inputs resident in HBM;
  roofline     for the dominant kernel (the fp64 trailing-update GEMM):
               algorithmic flops per launch / mean launch time from HIP events
               recorded on the launch stream during the timed steps, against
               the MI355X fp64 matrix peak;
  parts        the same per workload and per kernel, including the batched
               kernel's effective HBM bandwidth against 8 TB/s; after the
               timed steps, the other configurations (fp64 64 x 64; fp32
               4096^2, alpha 0.5; complex fp64 8192 x 2048) and the fp64
               8192^2 solve at every block size, each by the pages' protocol
               (one warm-up, mean of the next 9) with the per-phase split of
               the pages' Table 3;
  cpu_baseline the CPU oracle timed on a bounded sample of the same workloads,
               on all host threads and (C1, C2 sample) on one core.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {  # MI355X published dense peaks
    "hbm_gbs": 8000.0,
    "fp64_mfma_tflops": 78.6,
    "fp32_mfma_tflops": 157.3,
}
METRIC = "TRSM GFLOP/s & % MFMA/HBM roofline (fp64 m=n=8192; batched 64×64 zd)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev(a):
    """Column-major numpy operand (2-D or batched) -> column-major device tensor."""
    import torch
    if a.ndim == 2:
        return torch.from_numpy(np.ascontiguousarray(a.T)).to("cuda").T
    return torch.from_numpy(np.ascontiguousarray(np.transpose(a, (0, 2, 1)))).to("cuda").transpose(1, 2)


def kernel_algorithmic(rec):
    """(flops, bytes) of one launch by its record, counted algorithmically:
    GEMM 2MNK (x4 complex); triangular solve GEMM M(M+1)N (x4 complex);
    small kernel: triangle of L + B read + X written per problem."""
    cplx = rec["dtype"] in (2, 3)
    es = {0: 4, 1: 8, 2: 16, 3: 8}[rec["dtype"]]
    f = 4.0 if cplx else 1.0
    m, n, k, b = rec["m"], rec["n"], rec["k"], rec["batch"]
    if rec["kind"] == "update_gemm":
        return 2.0 * m * n * k * f, es * (m * k + k * n + 2.0 * m * n)
    if rec["kind"] == "solve_gemm":
        return m * (m + 1.0) * n * f, es * (m * (m + 1) / 2.0 + 2.0 * m * n)
    if rec["kind"] == "small":
        return m * m * n * f * b, es * b * (m * (m + 1) / 2.0 + 2.0 * m * n)
    if rec["kind"] == "diag_inv":
        ib, nb = n, b
        return f * nb * ib ** 3 / 3.0, es * nb * (ib * (ib + 1) / 2.0 + ib * ib)
    if rec["kind"] == "copy":
        return 0.0, es * 2.0 * m * n
    return 0.0, 0.0


def summarize_kernels(records):
    out = {}
    for r in records:
        fl, by = kernel_algorithmic(r)
        d = out.setdefault(r["kind"] + {0: "_f32", 1: "_f64", 2: "_c64", 3: "_c32"}[r["dtype"]],
                           {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
        d["launches"] += 1
        d["ms"] += r["ms"]
        d["flops"] += fl
        d["bytes"] += by
    for d in out.values():
        s = d["ms"] * 1e-3
        d["mean_ms"] = d["ms"] / d["launches"]
        d["tflops"] = d["flops"] / s / 1e12 if s > 0 else None
        d["gbs"] = d["bytes"] / s / 1e9 if s > 0 else None
    return out


def update_tiles(records):
    """Macro tile of each fp64 update launch, by the library's rule for a
    single real fp64 product with 16-byte aligned operands (launch_sized in
    gemm_mfma.hip): 128 x 128 on the LDS-free kernel when M > 64 and that
    gives at least 512 tiles in rounds of 512 at least 3/4 full, 128 x 64
    when that gives at least 2048, 64 x 32 when 64 x 64 gives fewer than
    1024, 64 x 64 otherwise."""
    counts = {}
    for r in records:
        if r["kind"] != "update_gemm" or r["dtype"] != 1:
            continue
        M, N = r["m"], r["n"]
        t128 = -(-M // 128) * -(-N // 128)
        if M > 64 and t128 >= 512 and 4 * t128 >= 3 * 512 * -(-t128 // 512):
            t = "128x128 LDS-free (gemm_lf_kernel)"
        elif -(-M // 128) * -(-N // 64) >= 2048:
            t = "128x64"
        elif -(-M // 64) * -(-N // 64) < 1024:
            t = "64x32"
        else:
            t = "64x64"
        counts[t] = counts.get(t, 0) + 1
    return counts


def phase2_order(records):
    """Which phase-2 order the fp64 solve ran: right-looking updates all have
    K = ib, left-looking ones a K that grows by ib per block row."""
    ks = {r["k"] for r in records if r["kind"] == "update_gemm" and r["dtype"] == 1}
    return "right-looking" if len(ks) <= 1 else "left-looking"


def cpu_baseline(big, small, seconds=12.0):
    """Time the oracle (as it stands) on a bounded sample of each workload:
    about seconds/2 on a block of right-hand-side columns of the large solve
    (columns are independent, so the sample is a smaller instance of the same
    work) and about seconds/2 on repeats of the whole batched workload."""
    import oracle
    L4, B4, a4, cfg4 = big
    L2, B2, a2, cfg2 = small
    cores = oracle.num_threads()
    # calibrate on 64 columns, then size the column block to ~seconds/2
    t = time.perf_counter()
    oracle.solve(L4, np.asfortranarray(B4[:, :64]), a4)
    t64 = max(time.perf_counter() - t, 1e-3)
    ncols = int(min(cfg4.n, max(64, 64 * (seconds / 2) / t64)))
    t = time.perf_counter()
    oracle.solve(L4, np.asfortranarray(B4[:, :ncols]), a4)
    t_big = time.perf_counter() - t
    fl_big = float(cfg4.m) ** 2 * ncols
    t = time.perf_counter()
    oracle.solve_batched(L2, B2, a2)
    t1 = max(time.perf_counter() - t, 1e-3)
    reps = int(min(200, max(1, (seconds / 2) / t1)))
    t = time.perf_counter()
    for _ in range(reps):
        oracle.solve_batched(L2, B2, a2)
    t_small = time.perf_counter() - t
    fl_small = cfg2.flops * reps
    return {
        "value": (fl_big + fl_small) / (t_big + t_small) / 1e9,
        "unit": "GFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{cfg4.name}: {ncols} of {cfg4.n} right-hand-side columns at full m "
                   f"({t_big:.1f} s); {cfg2.name}: the whole batch {reps} times ({t_small:.1f} s)"),
        "big_gflops": fl_big / t_big / 1e9,
        "small_gflops": fl_small / t_small / 1e9,
    }


def measured_traffic(kernel_key):
    """HBM bytes per launch of `kernel_key` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when the summary is missing or
    was taken on a different version of the kernel's source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec["bytes_per_launch"]


PHASES = {"diag_inv": "diagonal inversion", "update_gemm": "GEMM update", "solve_gemm": "solve GEMM",
          "copy": "copy", "small": "direct solve", "fill": "zero fill"}


def protocol_time(T, call, restore, warm_s=0.3, runs=9):
    """The pages' protocol (HSMA-TRSM section 5.1: one warm-up run, then the
    mean of the next 9), after a sustained warm-up of about warm_s seconds of
    the same call (the GPU clock drops while the host prepares inputs).  B is
    restored from a pristine copy outside the timed events.  Also returns the
    launch records of the timed runs (per-phase split, section 5.3.1
    Table 3)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        restore()
        call()
    restore()
    call()  # the protocol's own warm-up run
    torch.cuda.synchronize()
    ts = []
    for _ in range(runs):
        restore()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    # per-launch records from separate runs: two event records around each
    # of a solve's launches lengthen a short solve measurably (fp32 4096^2,
    # 17 launches: 0.71 -> 0.78 ms), so the timed runs above take none
    T.trsm_profile_select(None)
    T.trsm_profile_start()
    for _ in range(3):
        restore()
        call()
    torch.cuda.synchronize()
    T.trsm_profile_stop()
    return sum(ts) / len(ts), min(ts), T.profile_records()


def phase_split(records):
    """Share of kernel time per phase (diagonal inversion, GEMM update, solve
    GEMM, copy), as the pages' Table 3 reports it."""
    tot = sum(r["ms"] for r in records) or 1.0
    out = {}
    for r in records:
        k = PHASES.get(r["kind"], r["kind"])
        out[k] = out.get(k, 0.0) + r["ms"] / tot
    return {k: round(v, 4) for k, v in out.items()}


def time_other_configs(T, to_dev_fn, a4d, b4_host, a4, cfg4):
    """C1, C3 and C5 on their own and C4 at every block size, by the pages'
    protocol.  Returns bench 'parts' entries."""
    import torch
    from trsm_inputs import CONFIGS, make_config
    parts = []
    peak = {"f32": PEAK["fp32_mfma_tflops"], "f64": PEAK["fp64_mfma_tflops"], "c64": PEAK["fp64_mfma_tflops"]}

    def entry(cfg, mean_ms, min_ms, recs, **extra):
        tf = cfg.flops / (mean_ms * 1e-3) / 1e12
        e = {"workload": cfg.name, "protocol": "1 warm-up + mean of 9", "mean_ms": mean_ms, "min_ms": min_ms,
             "tflops": tf, f"frac_{'fp32' if cfg.dtype == 'f32' else 'fp64'}_mfma_peak": tf / peak[cfg.dtype]}
        if cfg.m > 64:
            e["phases"] = phase_split(recs)
            kern = summarize_kernels(recs)
            e["kernels"] = {k: {"mean_ms": v["mean_ms"], "launches_per_solve": v["launches"] / 3,
                                "tflops": v["tflops"]} for k, v in kern.items()}
        e.update(extra)
        return e

    for name in ("c1_f64_64", "c3_f32_4096", "c5_c64_8192x2048"):
        cfg = CONFIGS[name]
        log(f"{name}: inputs and timing")
        L, B, a = make_config(cfg)
        Ad, B0 = to_dev_fn(L), to_dev_fn(B)
        Bd = B0.clone()
        del L, B
        # one second of the same call first: the clock drops while the host
        # draws the inputs, and 0.3 s did not bring it back (C3 read 0.78 ms
        # where it runs 0.71 ms in steady state)
        mean_ms, min_ms, recs = protocol_time(T, lambda: T.trsm_lln(Ad, Bd, a), lambda: Bd.copy_(B0),
                                              warm_s=1.0)
        extra = {}
        if cfg.m > 64:
            extra["ib"] = T.trsm_lln_select_ib({"f32": T.R32F, "f64": T.R64F, "c64": T.C64F}[cfg.dtype],
                                               cfg.m, cfg.n)
        else:
            # latency: back-to-back calls on the stream, solved in place
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(200):
                T.trsm_lln(Ad, Bd, a)
            e1.record()
            torch.cuda.synchronize()
            extra["us_per_call_back_to_back"] = e0.elapsed_time(e1) * 1e3 / 200
        parts.append(entry(cfg, mean_ms, min_ms, recs, **extra))
        del Ad, B0, Bd
        torch.cuda.empty_cache()

    # C4 at each block size of the sweep (section 4.3.2), the table's choice marked
    B0 = to_dev_fn(b4_host)
    Bd = B0.clone()
    table_ib = T.trsm_lln_select_ib(T.R64F, cfg4.m, cfg4.n)
    for ib in (64, 128, 256, 512, 1024):
        log(f"{cfg4.name} at ib {ib}")
        mean_ms, min_ms, recs = protocol_time(T, lambda: T.trsm_lln_ex(a4d, Bd, a4, ib=ib),
                                              lambda: Bd.copy_(B0), warm_s=0.1)
        parts.append(entry(cfg4, mean_ms, min_ms, recs, ib=ib, table_choice=(ib == table_ib)))
    del B0, Bd
    torch.cuda.empty_cache()
    return parts


SINGLE_CORE = r"""
import json, sys, time
sys.path.insert(0, {root!r})
import numpy as np
import oracle
from trsm_inputs import CONFIGS, make_config
out = {{"threads": oracle.num_threads()}}
cfg = CONFIGS["c1_f64_64"]
L, B, a = make_config(cfg)
oracle.solve(L, B, a)
reps, t = 0, time.perf_counter()
while time.perf_counter() - t < {c1_s}:
    oracle.solve(L, B, a)
    reps += 1
dt = time.perf_counter() - t
out["c1"] = {{"gflops": cfg.flops * reps / dt / 1e9, "us_per_solve": dt / reps * 1e6, "solves": reps}}
cfg = CONFIGS["c2_c64_64x64_b8192"]
L, B, a = make_config(cfg)
nb = {c2_problems}
Ls, Bs = L[:nb], B[:nb]
oracle.solve_batched(Ls, Bs, a)
reps, t = 0, time.perf_counter()
while time.perf_counter() - t < {c2_s}:
    oracle.solve_batched(Ls, Bs, a)
    reps += 1
dt = time.perf_counter() - t
fl = cfg.flops / cfg.batch * nb * reps
out["c2"] = {{"gflops": fl / dt / 1e9, "solves_per_s": nb * reps / dt, "problems": nb, "repeats": reps}}
print(json.dumps(out))
"""


def cpu_single_core(c1_s=1.5, c2_s=4.0, c2_problems=512):
    """The oracle on one host core (OMP_NUM_THREADS=1, in a child process so
    the thread count is fixed before OpenMP starts) on C1 and on the first
    c2_problems problems of C2, repeated for about c1_s and c2_s seconds."""
    import subprocess
    code = SINGLE_CORE.format(root=ROOT, c1_s=c1_s, c2_s=c2_s, c2_problems=c2_problems)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        log(f"single-core oracle run failed: {r.stderr[-500:]}")
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the sampled residual check")
    ap.add_argument("--ib", type=int, default=0, help="force the diagonal block size of the fp64 solve")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing C1, C3, C5 and the per-block-size C4 rows after the timed steps")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the solve shards by right-hand-side columns; see the design notes). "
              f"Asked for --gpus {args.gpus} / WORLD_SIZE {world}.", file=sys.stderr)
        sys.exit(2)

    import torch

    import triangular_solve_trsm_amd as T
    from trsm_inputs import CONFIGS, make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg4 = CONFIGS["c4_f64_8192"]
    cfg2 = CONFIGS["c2_c64_64x64_b8192"]
    log("generating inputs")
    L4, B4, a4 = make_config(cfg4)
    L2, B2, a2 = make_config(cfg2)
    A4d, B4d = to_dev(L4), to_dev(B4)
    A2d, B2d = to_dev(L2), to_dev(B2)
    torch.cuda.synchronize()

    marks = []  # (event before C4, between, after C2) per timed step

    def step(mark=False):
        if mark:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
        if args.ib:
            T.trsm_lln_ex(A4d, B4d, a4, ib=args.ib)
        else:
            T.trsm_lln(A4d, B4d, a4)
        if mark:
            ev[1].record()
        T.trsm_lln_strided_batched(A2d, B2d, a2)
        if mark:
            ev[2].record()
            marks.append(ev)

    parity = None
    if not args.no_check:
        # Sanity check of the first solve by its residual ||L X - alpha B|| on
        # sampled right-hand sides, computed with torch on the GPU (the oracle
        # is not used here; the test suite holds the parity tests).
        log("residual check on sampled columns / problems")
        step()
        torch.cuda.synchronize()
        cols = torch.as_tensor(np.unique(np.linspace(0, cfg4.n - 1, 8).astype(int)), device="cuda")
        L4t = torch.tril(A4d.contiguous())
        X4 = B4d[:, cols].contiguous()
        B4s = to_dev(B4)[:, cols].contiguous()
        r4 = (torch.linalg.norm(L4t @ X4 - a4 * B4s) /
              (torch.linalg.norm(L4t) * torch.linalg.norm(X4) + abs(a4) * torch.linalg.norm(B4s))).item()
        del L4t
        probs = torch.arange(0, cfg2.batch, 97, device="cuda")
        L2t = torch.tril(A2d[probs].contiguous())
        X2 = B2d[probs].contiguous()
        B2s = to_dev(B2)[probs].contiguous()
        r2 = (torch.linalg.norm(torch.bmm(L2t, X2) - a2 * B2s) /
              (torch.linalg.norm(L2t) * torch.linalg.norm(X2) + abs(a2) * torch.linalg.norm(B2s))).item()
        parity = {"c4_sampled_cols_residual": r4, "c2_sampled_problems_residual": r2}
        log(f"residuals: {parity}")
        if not (r4 <= 10 * cfg4.m * 2.0 ** -53 and r2 <= 10 * cfg2.m * 2.0 ** -53):
            raise SystemExit(f"residual check failed: {parity}")
        B4d.copy_(to_dev(B4))
        B2d.copy_(to_dev(B2))
        torch.cuda.synchronize()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # HIP events around the dominant kernel's launches (and the batched small
    # solve's, for its HBM figure) only: events around every launch would
    # lengthen the step they measure
    T.trsm_profile_select(["update_gemm", "small"])
    T.trsm_profile_start()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step(mark=True)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    T.trsm_profile_stop()
    recs = T.profile_records()
    ev_ms = ev0.elapsed_time(ev1)
    log(f"timed region: {wall * 1e3:.2f} ms wall, {ev_ms:.2f} ms events, {len(recs)} launches")

    kern = summarize_kernels(recs)
    flops_step = cfg4.flops + cfg2.flops
    value = flops_step * args.steps / wall / 1e9
    upd = kern.get("update_gemm_f64", {})
    small = kern.get("small_c64", {})
    c4_ms = sum(e[0].elapsed_time(e[1]) for e in marks) / len(marks)
    c2_ms = sum(e[1].elapsed_time(e[2]) for e in marks) / len(marks)

    roofline = {
        "bound": "mfma",
        "kernel": "update_gemm_f64 (launches per tile: "
                  + ", ".join(f"{t} x{c // args.steps}" for t, c in sorted(update_tiles(recs).items()))
                  + f" per step; {phase2_order(recs)} phase 2)",
        "achieved": upd.get("tflops"),
        "peak": PEAK["fp64_mfma_tflops"],
        "unit": "TFLOP/s",
        "frac": (upd.get("tflops") or 0.0) / PEAK["fp64_mfma_tflops"],
        "traffic": measured_traffic("update_gemm_f64"),
        "launches": upd.get("launches"),
        "mean_launch_ms": upd.get("mean_ms"),
    }
    parts = [
        {"workload": cfg4.name, "ms_per_step": c4_ms, "gflops": cfg4.flops / (c4_ms * 1e-3) / 1e9 if c4_ms else None,
         "frac_fp64_mfma_peak": cfg4.flops / (c4_ms * 1e-3) / 1e12 / PEAK["fp64_mfma_tflops"] if c4_ms else None,
         "ib": args.ib or T.trsm_lln_select_ib(T.R64F, cfg4.m, cfg4.n)},
        {"workload": cfg2.name, "ms_per_step": c2_ms,
         "gflops": cfg2.flops / (c2_ms * 1e-3) / 1e9 if c2_ms else None,
         "solves_per_s": cfg2.batch / (c2_ms * 1e-3) if c2_ms else None,
         "hbm_gbs": small.get("gbs"), "frac_hbm_peak": (small.get("gbs") or 0.0) / PEAK["hbm_gbs"],
         "roofline_bound": "hbm"},
    ]

    if not args.no_other_configs:
        parts += time_other_configs(T, to_dev, A4d, B4, a4, cfg4)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        cpu = cpu_baseline((L4, B4, a4, cfg4), (L2, B2, a2, cfg2))
        log(f"cpu baseline: {cpu['value']:.2f} GFLOP/s on {cpu['cores']} threads")
        log("cpu baseline on one core (C1, C2 sample)")
        cpu["single_core"] = cpu_single_core()

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "fp64 TRSM m=n=8192 (alpha=1) + complex-fp64 TRSM batch 8192 x (64x64) (alpha=1)",
                   "layout": "column-major, lda=ldb=m", "seeds": [cfg4.seed, cfg2.seed]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parts": parts,
        "kernels": kern,
        "events_ms_per_step": ev_ms / args.steps,
        "residual_check": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
