"""Parity of the HIP library with the CPU oracle on the GPU.

Every case calls the C ABI through the Python binding and compares with the
oracle element by element: normwise relative error <= 1e-12 (fp64, complex
fp64) or <= 1e-4 (fp32), the bar fixed for this operation.  Well-conditioned
inputs put correct results near 1e-16 / 1e-7 (the pages' Table 2 scale); a
sanity bound of 1e-13 / 1e-5 is checked as well so that a result near the
tolerance (a sign of a bug) does not pass silently.

Full-size workloads are checked on sampled right-hand-side columns (columns
are independent: column j of X depends only on L and column j of B) and, on
the whole output, by the residual property ||L X - alpha B|| that holds at
any size.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from gpu_util import CPLX, TOL, from_dev, ld_of, max_problem_nrel, nrel, to_dev, torch_dtype
from trsm_inputs import CONFIGS, make_config, make_problem, small_integer_rhs, unit_bidiagonal_minus_one

pytestmark = pytest.mark.gpu

SANITY = {"f32": 1e-5, "f64": 1e-13, "c64": 1e-13, "c32": 1e-5}


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import triangular_solve_trsm_amd as T
    return T


def sync():
    import torch
    torch.cuda.synchronize()


def solve_gpu(T, L, B, alpha, **kw):
    Ad = to_dev(L)
    Bd = to_dev(B)
    if kw:
        T.trsm_lln_ex(Ad, Bd, alpha, **kw)
    else:
        T.trsm_lln(Ad, Bd, alpha)
    sync()
    return from_dev(Bd)


def check(dtype, X, ref, what=""):
    e = nrel(X, ref)
    assert e <= TOL[dtype], f"{what}: error {e:.3e} > {TOL[dtype]}"
    assert e <= SANITY[dtype], f"{what}: error {e:.3e} is within tolerance but far above rounding"
    return e


# ---- the five workloads ----------------------------------------------------

def test_c1_single_f64_64(T):
    cfg = CONFIGS["c1_f64_64"]
    L, B, a = make_config(cfg)
    check("f64", solve_gpu(T, L, B, a), oracle.solve(L, B, a), cfg.name)


def test_c2_batched_c64_64(T):
    cfg = CONFIGS["c2_c64_64x64_b8192"]
    L, B, a = make_config(cfg)
    Ad, Bd = to_dev(L), to_dev(B)
    T.trsm_lln_strided_batched(Ad, Bd, a)
    sync()
    X = from_dev(Bd)
    ref = oracle.solve_batched(L, B, a)
    e = max_problem_nrel(X, ref)
    assert e <= TOL["c64"] and e <= SANITY["c64"], e


def tile_columns(n, width=64):
    """One column in every `width`-column tile of B (its position inside the
    tile varies, so every lane position of the GEMM tiles is met), plus the
    last column."""
    cols = [t * width + (t * 37) % width for t in range((n + width - 1) // width)]
    return np.unique(np.array([c for c in cols if c < n] + [n - 1]))


@pytest.mark.parametrize("name", ["c3_f32_4096", "c4_f64_8192", "c5_c64_8192x2048"])
def test_large_workloads_vs_oracle_and_residual(T, name):
    """C3 is compared with the oracle on its whole output; C4 and C5 on one
    column of every 64-column tile plus the last (columns are independent
    problems), 129 and 33 columns.  The whole output of each also goes
    through the residual bound."""
    import torch
    cfg = CONFIGS[name]
    L, B, a = make_config(cfg)
    Ad, Bd = to_dev(L), to_dev(B)
    B0 = Bd.clone()
    T.trsm_lln(Ad, Bd, a)
    sync()
    if name == "c3_f32_4096":
        check(cfg.dtype, from_dev(Bd), oracle.solve(L, B, a), name + " (whole output)")
    else:
        cols = tile_columns(cfg.n)
        Xs = from_dev(Bd[:, torch.as_tensor(cols, device=Bd.device)])
        ref = oracle.solve(L, np.asfortranarray(B[:, cols]), a)
        check(cfg.dtype, Xs, ref, f"{name} ({len(cols)} columns)")
    # residual of the whole output, computed on the GPU in float64/complex128
    wide = torch.complex128 if cfg.dtype == "c64" else torch.float64
    Lw = torch.tril(Ad.to(wide))
    Xw, Bw = Bd.to(wide), B0.to(wide)
    R = Lw @ Xw - a * Bw
    res = (torch.linalg.norm(R) / (torch.linalg.norm(Lw) * torch.linalg.norm(Xw)
                                   + abs(a) * torch.linalg.norm(Bw))).item()
    u = 2.0 ** -24 if cfg.dtype == "f32" else 2.0 ** -53
    assert res <= 10 * cfg.m * u, res


MID_SHAPES = [("f64", 4096, 4096), ("f64", 2048, 2048), ("f64", 4096, 2048), ("f64", 8192, 1024),
              ("c64", 2048, 2048), ("c64", 4096, 2048), ("c64", 8192, 1024),
              ("f32", 8192, 8192), ("f32", 4096, 2048), ("f32", 2048, 2048),
              ("c32", 4096, 4096), ("c32", 8192, 2048), ("c32", 2048, 2048)]


@pytest.mark.parametrize("schedule", ["left", "right"])
@pytest.mark.parametrize("dtype,m,n", MID_SHAPES)
def test_mid_size_solves_vs_oracle(T, dtype, m, n, schedule, monkeypatch):
    """Whole solves at the table's block size whose products take the
    LDS-free forms for 64 to 511 tiles (half- and quarter-width workgroups,
    the K-split fp32 update, the complex fp32 mode, the complex triangular
    forms and the inversion's larger batched products), in both phase-2
    orders: one column of every 64-column tile plus the last against the
    oracle, and the whole output through the residual bound."""
    import torch
    monkeypatch.setenv("TRSM_SCHEDULE", schedule)
    print(f"case {dtype} m={m} n={n} {schedule}", flush=True)
    L, B = make_problem(dtype, m, n, seed=m + n + (schedule == "left"))
    a = 0.5 + 0.25j if dtype in CPLX else 0.5
    Ad, Bd = to_dev(L), to_dev(B)
    B0 = Bd.clone()
    T.trsm_lln(Ad, Bd, a)
    sync()
    cols = tile_columns(n)
    Xs = from_dev(Bd[:, torch.as_tensor(cols, device=Bd.device)])
    check(dtype, Xs, oracle.solve(L, np.asfortranarray(B[:, cols]), a), f"{dtype} {m}x{n} {schedule}")
    wide = torch.complex128 if dtype in CPLX else torch.float64
    Lw = torch.tril(Ad.to(wide))
    Xw, Bw = Bd.to(wide), B0.to(wide)
    res = (torch.linalg.norm(Lw @ Xw - a * Bw) / (torch.linalg.norm(Lw) * torch.linalg.norm(Xw)
                                                 + abs(a) * torch.linalg.norm(Bw))).item()
    u = 2.0 ** -24 if dtype in ("f32", "c32") else 2.0 ** -53
    assert res <= 10 * m * u, res


# ---- regime edges, ragged blocks, layouts ----------------------------------

EDGE_M = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129]
EDGE_N = [1, 5, 64, 65, 130]


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_regime_edges(T, dtype):
    worst = 0.0
    for m in EDGE_M:
        for n in EDGE_N:
            L, B = make_problem(dtype, m, n, seed=1000 + 7 * m + n)
            a = 0.5 - 0.25j if dtype in CPLX else 0.5
            X = solve_gpu(T, L, B, a)
            worst = max(worst, check(dtype, X, oracle.solve(L, B, a), f"{dtype} m={m} n={n}"))
    print(f"{dtype} regime edges: worst error {worst:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("ib", [64, 128, 256, 512, 1024])
def test_every_block_size_ragged(T, dtype, ib):
    """m = 1000 is a multiple of no candidate block size (below 1024 it is
    one ragged block); n = 257 is ragged against the GEMM tiles."""
    m, n = 1000, 257
    L, B = make_problem(dtype, m, n, seed=ib)
    a = 0.75 + 0.5j if dtype in CPLX else 0.75
    X = solve_gpu(T, L, B, a, ib=ib)
    check(dtype, X, oracle.solve(L, B, a), f"{dtype} ib={ib}")


@pytest.mark.parametrize("schedule", ["left", "right"])
def test_f64_updates_on_128x128_tiles(T, schedule, monkeypatch):
    """fp64 solves with updates on the 128 x 128 tile (at least 512 tiles,
    rounds of 512 at least 3/4 full): right-looking m = 3300, n = 4000 at
    ib 256 (first update 3044 x 4000, 768 tiles; later ones fall back to
    smaller tiles) and left-looking m = 2200, n = 8100 at ib 1024 (first
    update 1024 x 8100, 512 tiles; the ragged last block row of 152 rows
    uses smaller ones).  Ragged row and column tiles."""
    monkeypatch.setenv("TRSM_SCHEDULE", schedule)
    m, n, ib = (3300, 4000, 256) if schedule == "right" else (2200, 8100, 1024)
    L, B = make_problem("f64", m, n, seed=31)
    X = solve_gpu(T, L, B, 0.75, ib=ib)
    check("f64", X, oracle.solve(L, B, 0.75), f"f64 {schedule} m={m} n={n} ib={ib}")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("schedule", ["left", "right"])
@pytest.mark.parametrize("ib", [128, 256])
def test_both_phase2_schedules(T, dtype, schedule, ib, monkeypatch):
    """Left-looking (each block row updated once with K = r*ib) and
    right-looking phase 2 forced in turn: m = 1000 leaves a ragged last block
    row, n = 257 a ragged column tile, alpha != 1 checks that the scaling is
    applied exactly once per element."""
    monkeypatch.setenv("TRSM_SCHEDULE", schedule)
    m, n = 1000, 257
    L, B = make_problem(dtype, m, n, seed=7 + ib)
    a = -1.25 + 0.5j if dtype in CPLX else -1.25
    X = solve_gpu(T, L, B, a, ib=ib)
    check(dtype, X, oracle.solve(L, B, a), f"{dtype} {schedule} ib={ib}")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("schedule", ["left", "right"])
@pytest.mark.parametrize("splitk", ["0", "1024", "65536"])
@pytest.mark.parametrize("n", [1, 37, 64])
def test_split_k_phase2(T, dtype, schedule, splitk, n, monkeypatch):
    """Narrow B: solve and update products with few output tiles are cut
    along K into chunks whose partial sums are reduced afterwards.  Split-K
    off (0), at the default workgroup target and at a target that splits
    every product to the smallest chunk; m = 2000 with ib = 512 gives split
    K = 512 solves, a ragged last block (K = 464) that cannot be split, and
    left-looking updates with K up to 1536."""
    monkeypatch.setenv("TRSM_SCHEDULE", schedule)
    monkeypatch.setenv("TRSM_SPLITK", splitk)
    m = 2000
    L, B = make_problem(dtype, m, n, seed=2000 + n)
    a = 0.75 - 0.5j if dtype in CPLX else 0.75
    X = solve_gpu(T, L, B, a, ib=512)
    check(dtype, X, oracle.solve(L, B, a), f"{dtype} {schedule} splitk={splitk} n={n}")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("schedule", ["left", "right"])
def test_split_k_odd_leading_dimensions(T, dtype, schedule, monkeypatch):
    """Split K with lda = m + 3 and ldb = m + 1: columns that are not
    16-byte aligned take the dword load path, the reduction writes through
    the odd ldb, A's NaN upper triangle and padding stay unread and B's
    padding rows untouched."""
    monkeypatch.setenv("TRSM_SCHEDULE", schedule)
    monkeypatch.setenv("TRSM_SPLITK", "65536")
    m, n = 1100, 40
    L, B = make_problem(dtype, m, n, seed=1100, lda=m + 3, ldb=m + 1, upper="nan")
    Ad = to_dev(L, pad=np.nan)
    Bd = to_dev(B, pad=777.0)
    T.trsm_lln_ex(Ad, Bd, 1.0, ib=256)
    sync()
    import torch
    full = from_dev(torch.as_strided(Bd, (ld_of(B), n), (1, ld_of(B))))
    assert np.all(full[m:] == 777.0), "padding rows of B were modified"
    Lz, _ = make_problem(dtype, m, n, seed=1100)
    check(dtype, full[:m], oracle.solve(Lz, np.asfortranarray(B), 1.0), f"{dtype} {schedule} odd ld")


@pytest.mark.parametrize("dtype", ["f64", "c32"])
def test_split_k_wide_b_keeps_unsplit_products(T, dtype, monkeypatch):
    """m = 272 at ib = 256, right-looking, n = 65536: the update of the last
    16 rows (K = 256) fits the partial-sum bound at two chunks, but the
    reduction's grid takes at most 65535 columns, so a large split-K target
    must leave it whole.  Checked on sampled columns (independent
    problems)."""
    import torch
    monkeypatch.setenv("TRSM_SCHEDULE", "right")
    monkeypatch.setenv("TRSM_SPLITK", "1000000")
    m, n = 272, 65536
    L, B = make_problem(dtype, m, n, seed=65536)
    Ad, Bd = to_dev(L), to_dev(B)
    T.trsm_lln_ex(Ad, Bd, 1.0, ib=256)
    sync()
    cols = np.array([0, 1, 31, 32, 32767, 65534, 65535])
    Xs = from_dev(Bd[:, torch.as_tensor(cols, device=Bd.device)])
    check(dtype, Xs, oracle.solve(L, np.asfortranarray(B[:, cols]), 1.0), f"{dtype} n=65536")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("schedule", ["left", "right"])
def test_split_k_bidiagonal_exact(T, dtype, schedule, monkeypatch):
    """The running-sum problem stays exact when K is split: every partial sum
    is a small integer, so the reduction of the chunks is exact too."""
    monkeypatch.setenv("TRSM_SCHEDULE", schedule)
    monkeypatch.setenv("TRSM_SPLITK", "65536")
    m = 2048
    L = unit_bidiagonal_minus_one(m, dtype)
    B = small_integer_rhs(m, 16, dtype, seed=m)
    X = solve_gpu(T, L, B, 1.0, ib=512)
    assert np.array_equal(X, np.cumsum(B, axis=0)), f"{dtype} {schedule}"


@pytest.mark.parametrize("ks", ["1", "0"])
@pytest.mark.parametrize("dtype", ["f64", "c64"])
@pytest.mark.parametrize("schedule", ["left", "right"])
@pytest.mark.parametrize("m,n,ib", [(2100, 48, 512), (3000, 64, 1024), (1300, 5, 256), (2048, 33, 1024)])
def test_split_k_inside_workgroup(T, dtype, schedule, m, n, ib, ks, monkeypatch):
    """Products that split K (narrow B, a long K) run in fp64 and complex
    fp64 as one launch whose waves split K inside a workgroup and add
    their sums through LDS in a fixed order (TRSM_GEMM_KS=0: batched
    partial products and a reduction kernel).  Both against the oracle,
    ragged last block rows and column tiles, both phase-2 orders, split-K
    forced on every product that can take it; the two forms agree to
    rounding."""
    monkeypatch.setenv("TRSM_SCHEDULE", schedule)
    monkeypatch.setenv("TRSM_SPLITK", "65536")
    monkeypatch.setenv("TRSM_GEMM_KS", ks)
    print(f"case {dtype} {schedule} m={m} n={n} ib={ib} ks={ks}", flush=True)
    L, B = make_problem(dtype, m, n, seed=m + 3 * n)
    a = 0.75 + 0.25j if dtype in CPLX else 0.75
    X = solve_gpu(T, L, B, a, ib=ib)
    check(dtype, X, oracle.solve(L, B, a), f"{dtype} {schedule} m={m} n={n} ib={ib} ks={ks}")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_m_4097_narrow(T, dtype):
    m, n = 4097, 19
    L, B = make_problem(dtype, m, n, seed=4097)
    X = solve_gpu(T, L, B, 1.0)
    check(dtype, X, oracle.solve(L, B, 1.0), f"{dtype} m=4097")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("m,n", [(50, 40), (700, 90)])
def test_padding_and_poisoned_upper_triangle(T, dtype, m, n):
    """A's strict upper triangle and its padding rows hold NaN and must not
    matter; B's padding rows must be left untouched."""
    L, B = make_problem(dtype, m, n, seed=m + n, lda=m + 13, ldb=m + 5, upper="nan")
    Ad = to_dev(L, pad=np.nan)
    Bd = to_dev(B, pad=12345.0)
    T.trsm_lln(Ad, Bd, 1.0)
    sync()
    import torch
    full = from_dev(torch.as_strided(Bd, (ld_of(B), n), (1, ld_of(B))))
    assert np.all(full[m:] == 12345.0), "padding rows of B were modified"
    Lz, _ = make_problem(dtype, m, n, seed=m + n)
    check(dtype, full[:m], oracle.solve(Lz, np.asfortranarray(B), 1.0), f"{dtype} padded")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_force_blocked_small_sizes(T, dtype):
    for m in (1, 17, 64):
        L, B = make_problem(dtype, m, 33, seed=m)
        X = solve_gpu(T, L, B, 2.0, ib=64, force_blocked=True)
        check(dtype, X, oracle.solve(L, B, 2.0), f"{dtype} blocked m={m}")


# ---- batches -----------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("batch,m,n", [(1, 64, 64), (7, 33, 70), (7, 64, 64), (3, 150, 20)])
def test_batched(T, dtype, batch, m, n):
    L, B = make_problem(dtype, m, n, seed=batch * 100 + m, batch=batch)
    a = 0.5 - 0.25j if dtype in CPLX else -0.5
    Ad, Bd = to_dev(L), to_dev(B)
    T.trsm_lln_strided_batched(Ad, Bd, a)
    sync()
    X = from_dev(Bd)
    ref = oracle.solve_batched(L, B, a)
    e = max_problem_nrel(X, ref)
    assert e <= TOL[dtype] and e <= SANITY[dtype], e


# ---- special values and exact cases ------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("m", [40, 300])
def test_alpha_zero_zeroes_B_without_reading_A(T, dtype, m):
    import torch
    _, B = make_problem(dtype, m, 9, seed=2)
    Ad = to_dev(np.full((m, m), np.nan, dtype=B.dtype, order="F"))
    Bd = to_dev(B)
    T.trsm_lln(Ad, Bd, 0.0)
    sync()
    assert torch.all(Bd == 0).item()


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("m,ib", [(64, 0), (600, 128), (1000, 256)])
def test_bidiagonal_exact(T, dtype, m, ib):
    """Unit bidiagonal L with -1 below the diagonal: X is the running sum of
    B down each column, exact for integer B on every path (the inverse of
    each diagonal block is the all-ones lower triangle, also exact)."""
    L = unit_bidiagonal_minus_one(m, dtype)
    B = small_integer_rhs(m, 70, dtype, seed=m)
    X = solve_gpu(T, L, B, 1.0, ib=ib) if ib else solve_gpu(T, L, B, 1.0)
    assert np.array_equal(X, np.cumsum(B, axis=0)), f"{dtype} m={m}"


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("m,n,ib", [(40, 20, 0), (300, 50, 128), (1100, 70, 512)])
def test_zero_pivot_propagates_non_finite(T, dtype, m, n, ib):
    """No singularity check (BLAS convention): with l_kk = 0 the solve
    still completes; rows above k depend only on the leading k x k block and
    match the oracle, and every row from k down is non-finite, as in the
    oracle.  Direct path (m <= 64) and blocked path with the zero pivot
    inside a diagonal block."""
    k = m // 2 + 3
    L, B = make_problem(dtype, m, n, seed=77 + m)
    L = L.copy(order="F")
    L[k, k] = 0
    X = solve_gpu(T, L, B, 1.0, ib=ib) if ib else solve_gpu(T, L, B, 1.0)
    ref = oracle.solve(L, B, 1.0)
    assert np.all(~np.isfinite(ref[k:])), "oracle: rows from the zero pivot down are non-finite"
    assert np.all(np.isfinite(X[:k])), f"{dtype} m={m}: rows above the zero pivot must stay finite"
    check(dtype, X[:k], ref[:k], f"{dtype} m={m} rows above the zero pivot")
    assert np.all(~np.isfinite(X[k:])), f"{dtype} m={m}: rows from the zero pivot down must be non-finite"


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("m,n,ib", [(40, 20, 0), (300, 40, 128), (1100, 30, 512)])
def test_non_finite_b_entry_stays_in_its_column(T, dtype, m, n, ib):
    """A NaN in B at (k, j): every other column matches the oracle; in
    column j the rows of earlier diagonal blocks match the oracle and every
    row from k down is non-finite.  The rows between the start of k's block
    and k may also turn NaN (the method multiplies the block by its inverse,
    whose zeros above the diagonal meet the NaN); those that stay finite
    match the oracle.  Block: the 16-row panel on the direct path, ib rows
    on the blocked path."""
    k, j = m // 2 + 5, n // 3
    L, B = make_problem(dtype, m, n, seed=91 + m)
    B = B.copy(order="F")
    B[k, j] = np.nan
    X = solve_gpu(T, L, B, 1.0, ib=ib) if ib else solve_gpu(T, L, B, 1.0)
    ref = oracle.solve(L, B, 1.0)
    others = [c for c in range(n) if c != j]
    check(dtype, X[:, others], ref[:, others], f"{dtype} m={m}: columns without the NaN")
    start = (k // (ib if ib else 16)) * (ib if ib else 16)
    col, rcol = X[:, j], ref[:, j]
    assert np.all(np.isfinite(col[:start])), f"{dtype} m={m}: rows of earlier blocks must stay finite"
    if start:
        check(dtype, col[:start], rcol[:start], f"{dtype} m={m}: column {j} above the NaN's block")
    assert np.all(~np.isfinite(col[k:])), f"{dtype} m={m}: rows from the NaN down must be non-finite"
    fin = np.isfinite(col[start:k])
    if fin.any():
        check(dtype, col[start:k][fin], rcol[start:k][fin], f"{dtype} m={m}: finite rows of the NaN's block")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_deterministic(T, dtype):
    L, B = make_problem(dtype, 900, 300, seed=5)
    X1 = solve_gpu(T, L, B, 1.0)
    X2 = solve_gpu(T, L, B, 1.0)
    assert np.array_equal(X1, X2)


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_error_scale_vs_pages_table2(T, dtype):
    """At m = n = 1024 the GPU-vs-oracle error is of the order the pages
    report against a vendor TRSM (Table 2), at most 10x that figure."""
    import json
    here = os.path.dirname(os.path.abspath(__file__))
    table = json.load(open(os.path.join(here, "golden", "table2_normwise_error.json")))
    ref_err = table["error"][dtype][table["sizes"].index(1024)]
    L, B = make_problem(dtype, 1024, 1024, seed=1024)
    e = nrel(solve_gpu(T, L, B, 1.0), oracle.solve(L, B, 1.0))
    assert e <= 10 * ref_err, (dtype, e, ref_err)


def test_non_default_stream(T):
    import torch
    L, B = make_problem("f64", 500, 100, seed=3)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Ad, Bd = to_dev(L), to_dev(B)
        T.trsm_lln(Ad, Bd, 1.0, stream=s)
    s.synchronize()
    check("f64", from_dev(Bd), oracle.solve(L, B, 1.0), "side stream")


def test_current_stream_is_used(T):
    """With no stream argument a call goes to torch's current stream (the
    binding reads its raw handle for the operands' device)."""
    import torch
    dev = torch.cuda.current_device()
    L, B = make_problem("f64", 500, 100, seed=4)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert T._stream_handle(None, dev) == s.cuda_stream
        Ad, Bd = to_dev(L), to_dev(B)
        T.trsm_lln(Ad, Bd, 1.0)
    s.synchronize()
    check("f64", from_dev(Bd), oracle.solve(L, B, 1.0), "current stream")
    assert T._stream_handle(None, dev) == torch.cuda.current_stream().cuda_stream


def test_workspace_allocation_failure_leaves_B_untouched(T, monkeypatch):
    import torch
    L, B = make_problem("f64", 300, 40, seed=9)
    s = torch.cuda.Stream()  # fresh stream: its workspace is not cached yet
    with torch.cuda.stream(s):
        Ad, Bd = to_dev(L), to_dev(B)
    s.synchronize()
    monkeypatch.setenv("TRSM_FAIL_ALLOC", "1")
    with pytest.raises(T.TrsmError) as ei:
        T.trsm_lln(Ad, Bd, 1.0, stream=s)
    assert ei.value.status == 2
    monkeypatch.delenv("TRSM_FAIL_ALLOC")
    s.synchronize()
    assert np.array_equal(from_dev(Bd), B)
    T.trsm_lln(Ad, Bd, 1.0, stream=s)
    s.synchronize()
    check("f64", from_dev(Bd), oracle.solve(L, B, 1.0), "after failed alloc")
    T.trsm_release_workspace()


# ---- large batches: many resident workgroups per CU (fp64 / complex) --------

@pytest.mark.parametrize("dtype", ["f64", "c64", "c32"])
@pytest.mark.parametrize("batch,m,n", [(600, 64, 64), (600, 1, 64), (600, 17, 5), (520, 33, 100),
                                       (2100, 64, 64), (300, 48, 130)])
def test_batched_many_workgroups(T, dtype, batch, m, n):
    """Enough workgroups (problem x 64-column group) for several to be
    resident on every CU at once and for more than one round; ragged m,
    several column groups."""
    L, B = make_problem(dtype, m, n, seed=batch + 7 * m + n, batch=batch)
    a = 0.5 - 0.25j if dtype in CPLX else -0.75
    Ad, Bd = to_dev(L), to_dev(B)
    T.trsm_lln_strided_batched(Ad, Bd, a)
    sync()
    X = from_dev(Bd)
    ref = oracle.solve_batched(L, B, a)
    e = max_problem_nrel(X, ref)
    assert e <= TOL[dtype] and e <= SANITY[dtype], e


@pytest.mark.parametrize("dtype", ["f64", "c64", "c32"])
def test_batched_many_padded_nan_upper(T, dtype):
    """Padded leading dimensions, a NaN strict upper triangle and NaN padding
    in A; B's padding rows must stay untouched."""
    import torch
    batch, m, n = 700, 40, 70
    L, B = make_problem(dtype, m, n, seed=11, batch=batch, lda=m + 3, ldb=m + 5, upper="nan")
    Ad = to_dev(L, pad=np.nan)
    Bd = to_dev(B, pad=777.0)
    T.trsm_lln_strided_batched(Ad, Bd, 1.0)
    sync()
    ldb = m + 5
    full = from_dev(torch.as_strided(Bd, (batch, ldb, n), (Bd.stride(0), 1, ldb)))
    assert np.all(full[:, m:] == 777.0), "padding rows of B were modified"
    Lz, _ = make_problem(dtype, m, n, seed=11, batch=batch)
    ref = oracle.solve_batched(Lz, np.ascontiguousarray(B), 1.0)
    e = max_problem_nrel(full[:, :m], ref)
    assert e <= TOL[dtype] and e <= SANITY[dtype], e


@pytest.mark.parametrize("dtype", ["f64", "c64", "c32"])
def test_batched_many_bidiagonal_exact(T, dtype):
    """Unit bidiagonal L with -1 below the diagonal on every problem: X is the
    running column sum of integer B, exact on the batched direct path."""
    batch, m, n = 600, 64, 64
    L1 = unit_bidiagonal_minus_one(m, dtype)
    L = np.ascontiguousarray(np.broadcast_to(L1, (batch, m, m)).transpose(0, 2, 1)).transpose(0, 2, 1)
    Bs = np.stack([small_integer_rhs(m, n, dtype, seed=p) for p in range(batch)])
    B = np.ascontiguousarray(Bs.transpose(0, 2, 1)).transpose(0, 2, 1)
    Ad, Bd = to_dev(L), to_dev(B)
    T.trsm_lln_strided_batched(Ad, Bd, 1.0)
    sync()
    assert np.array_equal(from_dev(Bd), np.cumsum(B, axis=1))


# ---- guard regions around B ----------------------------------------------------

GUARD = 4096  # elements before and after B's storage


def guarded(a, ld, batch_stride=None):
    """Device buffer holding [GUARD sentinels][B storage][GUARD sentinels];
    returns (view of B, buffer, first element past B's storage)."""
    import torch
    dt = torch_dtype({np.float32: "f32", np.float64: "f64", np.complex128: "c64",
                      np.complex64: "c32"}[a.dtype.type])
    if a.ndim == 2:
        m, n = a.shape
        size = ld * n
    else:
        b, m, n = a.shape
        size = batch_stride * (b - 1) + ld * n
    buf = torch.full((GUARD + size + GUARD,), 4321.0, dtype=dt, device="cuda")
    if a.ndim == 2:
        view = torch.as_strided(buf, (m, n), (1, ld), GUARD)
    else:
        view = torch.as_strided(buf, (a.shape[0], m, n), (batch_stride, 1, ld), GUARD)
    view.copy_(torch.from_numpy(np.ascontiguousarray(a)).to("cuda"))
    return view, buf, GUARD + size


def guards_intact(buf, end):
    import torch
    return bool(torch.all(buf[:GUARD] == 4321.0).item()) and bool(torch.all(buf[end:] == 4321.0).item())


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("m,n,ib", [(64, 64, 0), (37, 130, 0), (700, 90, 128), (1000, 257, 0),
                                    (2100, 48, 512)])
def test_guard_regions_around_b_untouched(T, dtype, m, n, ib):
    """Nothing is written before B's first element or after its last one
    (element ldb*(n-1) + m - 1 and the padding after it) on the direct path,
    the blocked path (ragged tiles, split K at n = 48) and every type."""
    L, B = make_problem(dtype, m, n, seed=300 + m + n)
    a = 0.5 - 0.25j if dtype in CPLX else 0.5
    Ad = to_dev(L)
    Bd, buf, end = guarded(B, m + 3)
    if ib:
        T.trsm_lln_ex(Ad, Bd, a, ib=ib)
    else:
        T.trsm_lln(Ad, Bd, a)
    sync()
    assert guards_intact(buf, end), f"{dtype} m={m} n={n}: a guard region was written"
    check(dtype, from_dev(Bd), oracle.solve(L, B, a), f"{dtype} m={m} n={n} guarded")


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("batch,m,n", [(9, 64, 64), (5, 33, 70), (3, 150, 20)])
def test_guard_regions_around_batched_b_untouched(T, dtype, batch, m, n):
    """Batched problems at a stride with a gap after each problem's B: the
    gaps and the regions before the first and after the last problem keep
    their sentinels."""
    import torch
    L, B = make_problem(dtype, m, n, seed=batch + m, batch=batch)
    ldb = m + 2
    stride = ldb * n + 100
    Ad = to_dev(L)
    Bd, buf, end = guarded(B, ldb, stride)
    T.trsm_lln_strided_batched(Ad, Bd, 1.0)
    sync()
    assert guards_intact(buf, end)
    body = buf[GUARD:end]
    for p in range(batch - 1):  # the 100 elements after each problem but the last
        gap = body[p * stride + ldb * n: (p + 1) * stride]
        assert bool(torch.all(gap == 4321.0).item()), f"gap after problem {p} was written"
    full = from_dev(torch.as_strided(buf, (batch, ldb, n), (stride, 1, ldb), GUARD))
    assert np.all(full[:, m:] == 4321.0), "padding rows of B were modified"
    e = max_problem_nrel(full[:, :m], oracle.solve_batched(L, B, 1.0))
    assert e <= TOL[dtype] and e <= SANITY[dtype], e


@pytest.mark.parametrize("pc", ["0", "1"])
@pytest.mark.parametrize("batch,m,n", [(1, 64, 64), (7, 33, 70), (300, 64, 64), (1000, 50, 130),
                                       (257, 16, 1), (600, 64, 200)])
def test_batched_complex_both_small_kernels(T, pc, batch, m, n, monkeypatch):
    """Complex fp64 batches on each form of the direct solve, forced in
    turn (TRSM_SMALL_PC): the workgroup-per-task kernel and the persistent
    producer/consumer kernel (one workgroup per CU; a producer wave stages
    the next task's L and B in LDS and inverts its diagonal blocks while
    four MFMA waves solve the current task).  Fewer tasks than CUs, ragged m
    and n, several column groups per problem, and more tasks than
    workgroups."""
    monkeypatch.setenv("TRSM_SMALL_PC", pc)
    L, B = make_problem("c64", m, n, seed=batch + 3 * m + n, batch=batch, upper="nan")
    a = 0.5 - 0.25j
    Ad, Bd = to_dev(L), to_dev(B)
    T.trsm_lln_strided_batched(Ad, Bd, a)
    sync()
    Lz, _ = make_problem("c64", m, n, seed=batch + 3 * m + n, batch=batch)
    e = max_problem_nrel(from_dev(Bd), oracle.solve_batched(Lz, B, a))
    assert e <= TOL["c64"] and e <= SANITY["c64"], e
