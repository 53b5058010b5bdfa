"""Pins of the CPU oracle against facts that do not come from the oracle.

The oracle computes the forward-substitution formula of HSMA-TRSM ("Hierarchical
Shared Memory-Aware Optimization for TRSM on GPU Platforms", section 2.1 and
the equation of section 4.2.1).  None of these tests re-types that formula.
Each checks the oracle against something fixed independently of it:

* identity L: X = alpha B, bitwise;
* diagonal L: X = alpha B / d elementwise (two correctly rounded operations),
  bitwise;
* the unit bidiagonal L with -1 on the sub-diagonal, whose inverse is the
  all-ones lower triangle: X = alpha * (running column sums of B), exact for
  integer B, bitwise;
* exact rational arithmetic on tiny integer systems: with power-of-two
  diagonals the solution is a short dyadic rational, so L X - alpha B must be
  exactly zero; with other diagonals the result must sit within a few units
  in the last place of the exact solution found by Gauss-Jordan elimination
  on the full matrix (a different algorithm);
* the residual bound of a backward-stable solve;
* loop-order invariance (column order == row-wise dot order, bitwise);
* agreement with scipy's LAPACK/BLAS triangular solves;
* the error scale the pages report against a vendor TRSM (Table 2).

``test_planted_mistakes_are_caught`` compiles mutated copies of the oracle
(a flipped sign, a transposed operand, a dropped term, ...) and checks that
the quick pins reject every one of them.
"""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg as sla
from scipy.linalg import blas as sblas

import oracle
from trsm_inputs import (CONFIGS, diagonal, identity, make_config, make_problem,
                         small_integer_rhs, unit_bidiagonal_minus_one)

HERE = os.path.dirname(os.path.abspath(__file__))
DTYPES = ["f32", "f64", "c64", "c32"]
NP = {"f32": np.float32, "f64": np.float64, "c64": np.complex128, "c32": np.complex64}
UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "f64": 2.0 ** -53, "c64": 2.0 ** -53, "c32": 2.0 ** -24}
CPLX = ("c64", "c32")
SINGLE = ("f32", "c32")


def nrel(X, Xref):
    """Normwise relative difference ||X - Xref||_F / ||Xref||_F (0 if both are 0)."""
    Xref = np.asarray(Xref, dtype=np.complex128)
    d = np.linalg.norm(np.asarray(X, dtype=np.complex128) - Xref)
    r = np.linalg.norm(Xref)
    return d / r if r > 0 else d


def bits_equal(a, b):
    """Exact equality of every element (IEEE ==, so +0 and -0 are equal: the
    sign of an exact zero depends on whether a zero product was subtracted)."""
    a = np.asarray(a)
    b = np.asarray(b)
    return a.shape == b.shape and a.dtype == b.dtype and bool(np.all(a == b))


# ---------------------------------------------------------------------------
# quick pin checks, parametrised by an oracle build (used for mutants too)
# ---------------------------------------------------------------------------

def check_identity(orc, dtype):
    for m, n in [(1, 1), (7, 3), (64, 64), (130, 5)]:
        B = small_integer_rhs(m, n, dtype, seed=m * 31 + n)
        alphas = [1.0, 0.5, -2.0] + ([0.5 - 0.25j, -1j] if dtype in CPLX else [])
        for a in alphas:
            X = orc.solve(identity(m, dtype), B, a)
            expect = (np.asarray(a, dtype=NP[dtype]) * B).astype(NP[dtype])
            assert bits_equal(X, np.asfortranarray(expect)), (dtype, m, n, a)


def check_diagonal(orc, dtype):
    rng = np.random.default_rng(7)
    m, n = 37, 11
    # powers of two: every step is exact
    d = rng.choice([0.5, 1.0, 2.0, 4.0, -2.0, -0.25], size=m)
    B = small_integer_rhs(m, n, dtype, seed=3)
    for a in [1.0, -0.5] + ([0.5 - 0.25j] if dtype in CPLX else []):
        X = orc.solve(diagonal(d, dtype), B, a)
        aB = np.asarray(a, dtype=NP[dtype]) * B
        if dtype in CPLX:
            expect = aB.real / d[:, None] + 1j * (aB.imag / d[:, None])
        else:
            expect = aB / d[:, None].astype(NP[dtype])
        assert bits_equal(X, np.asfortranarray(expect.astype(NP[dtype]))), (dtype, a)
    # general diagonal: alpha*b rounded, then one correctly rounded division
    d = rng.uniform(1.0, 2.0, m).astype(np.float32 if dtype in SINGLE else np.float64)
    _, Bg = make_problem(dtype, m, n, seed=11)
    for a in [1.0, 0.7]:
        X = orc.solve(diagonal(d, dtype), Bg, a)
        aB = (np.asarray(a, dtype=NP[dtype]) * Bg).astype(NP[dtype])
        if dtype in CPLX:
            expect = aB.real / d[:, None] + 1j * (aB.imag / d[:, None])
        else:
            expect = aB / d[:, None]
        assert bits_equal(X, np.asfortranarray(expect.astype(NP[dtype]))), (dtype, a)
    if dtype in CPLX:
        # complex (non-real) diagonal: compare with numpy's complex division
        dz = (rng.uniform(1, 2, m) + 1j * rng.uniform(-1, 1, m)).astype(NP[dtype])
        X = orc.solve(np.asfortranarray(np.diag(dz)), Bg, 1.0)
        expect = Bg / dz[:, None]
        err = np.abs(X - expect) / np.abs(expect)
        assert err.max() < 8 * UNIT_ROUNDOFF[dtype], err.max()


def check_bidiagonal(orc, dtype):
    """Unit lower bidiagonal with -1 below the diagonal: L^{-1} is the
    all-ones lower triangle ((L T)_ij = [i>=j] - [i-1>=j] = delta_ij), so X is
    alpha times the running sums down each column of B."""
    for m, n in [(1, 3), (2, 2), (65, 9), (300, 4)]:
        L = unit_bidiagonal_minus_one(m, dtype)
        B = small_integer_rhs(m, n, dtype, seed=m + 5)
        for a in [1.0, 2.0] + ([1j] if dtype in CPLX else []):
            X = orc.solve(L, B, a)
            expect = np.asarray(a, dtype=NP[dtype]) * np.cumsum(B, axis=0)
            assert bits_equal(X, np.asfortranarray(expect.astype(NP[dtype]))), (dtype, m, a)


def _to_frac(x):
    if isinstance(x, (complex, np.complexfloating)):
        return (Fraction(float(x.real)), Fraction(float(x.imag)))
    return (Fraction(float(x)), Fraction(0))


def _cmul(a, b):
    return (a[0] * b[0] - a[1] * b[1], a[0] * b[1] + a[1] * b[0])


def exact_residual_is_zero(L, X, B, alpha):
    """L X - alpha B == 0 in exact rational arithmetic (complex as pairs)."""
    m, n = B.shape
    al = _to_frac(alpha)
    for j in range(n):
        for i in range(m):
            s = _cmul(al, _to_frac(B[i, j]))
            s = (-s[0], -s[1])
            for k in range(i + 1):
                p = _cmul(_to_frac(L[i, k]), _to_frac(X[k, j]))
                s = (s[0] + p[0], s[1] + p[1])
            if s != (0, 0):
                return False
    return True


def random_integer_lower(m, dtype, rng, diag_choices):
    d = rng.choice(diag_choices, size=m)
    if dtype in CPLX:
        off = rng.integers(-3, 4, (m, m)) + 1j * rng.integers(-3, 4, (m, m))
    else:
        off = rng.integers(-3, 4, (m, m))
    L = np.tril(off, -1) + np.diag(d)
    return np.asfortranarray(L.astype(NP[dtype]))


def check_exact_dyadic(orc, dtype):
    rng = np.random.default_rng(2024)
    for trial in range(12):
        m = int(rng.integers(1, 6 if dtype not in SINGLE else 4))
        n = int(rng.integers(1, 5))
        L = random_integer_lower(m, dtype, rng, [1.0, -1.0, 2.0, -2.0, 4.0])
        B = small_integer_rhs(m, n, dtype, seed=trial)
        for a in [1.0, -0.5] + ([0.5 + 0.5j] if dtype in CPLX else []):
            X = orc.solve(L, B, a)
            assert exact_residual_is_zero(L, X, B, a), (dtype, trial, a, L, B, X)


def gauss_jordan_exact(Lr, Br):
    """Exact solve of a general real system by Gauss-Jordan elimination with
    Fractions (pivot on the first nonzero entry).  Does not use the
    triangular structure."""
    m = len(Lr)
    M = [list(Lr[i]) + list(Br[i]) for i in range(m)]
    for c in range(m):
        p = next(r for r in range(c, m) if M[r][c] != 0)
        M[c], M[p] = M[p], M[c]
        piv = M[c][c]
        M[c] = [v / piv for v in M[c]]
        for r in range(m):
            if r != c and M[r][c] != 0:
                f = M[r][c]
                M[r] = [a - f * b for a, b in zip(M[r], M[c])]
    return [row[m:] for row in M]


def exact_solution(L, B, alpha):
    """Exact X for integer/dyadic inputs; complex via the real 2m x 2m
    embedding [[Re L, -Im L], [Im L, Re L]]."""
    m, n = B.shape
    aB = [[_cmul(_to_frac(alpha), _to_frac(B[i, j])) for j in range(n)] for i in range(m)]
    Lf = [[_to_frac(L[i, k]) for k in range(m)] for i in range(m)]
    if not np.iscomplexobj(L):
        Xr = gauss_jordan_exact([[Lf[i][k][0] for k in range(m)] for i in range(m)],
                                [[aB[i][j][0] for j in range(n)] for i in range(m)])
        return np.array([[float(v) for v in row] for row in Xr])
    big = [[Lf[i][k][0] for k in range(m)] + [-Lf[i][k][1] for k in range(m)] for i in range(m)]
    big += [[Lf[i][k][1] for k in range(m)] + [Lf[i][k][0] for k in range(m)] for i in range(m)]
    rhs = [[aB[i][j][0] for j in range(n)] for i in range(m)]
    rhs += [[aB[i][j][1] for j in range(n)] for i in range(m)]
    Xr = gauss_jordan_exact(big, rhs)
    return np.array([[complex(float(Xr[i][j]), float(Xr[m + i][j])) for j in range(n)]
                     for i in range(m)])


def check_scipy(orc, dtype):
    """scipy's LAPACK trtrs (solve_triangular) and BLAS trsm as independent
    implementations of the same operation."""
    tol = {"f32": 5e-6, "f64": 1e-14, "c64": 1e-14, "c32": 5e-6}[dtype]
    for (m, n, a) in [(64, 64, 1.0), (97, 33, 0.5), (200, 3, -1.5)] + (
            [(50, 20, 0.5 - 0.25j)] if dtype in CPLX else []):
        L, B = make_problem(dtype, m, n, seed=m * n)
        if dtype in CPLX:
            # make the diagonal genuinely complex so the complex division is exercised
            idx = np.arange(m)
            L = np.array(L, order="F")
            L[idx, idx] += 0.3j * np.cos(idx)
        X = orc.solve(L, B, a)
        aB = (np.asarray(a, dtype=NP[dtype]) * B).astype(NP[dtype])
        ref = sla.solve_triangular(np.array(L), aB, lower=True)
        assert nrel(X, ref) < tol, (dtype, m, n, a, nrel(X, ref))
        trsm = {"f32": sblas.strsm, "f64": sblas.dtrsm, "c64": sblas.ztrsm, "c32": sblas.ctrsm}[dtype]
        ref2 = trsm(a, np.array(L, order="F"), np.array(B, order="F"), side=0, lower=1,
                    trans_a=0, diag=0)
        assert nrel(X, ref2) < tol, (dtype, m, n, a, nrel(X, ref2))


def check_batched_matches_single(orc, dtype):
    L, B = make_problem(dtype, 23, 6, seed=99, batch=5)
    a = 0.5 - 0.25j if dtype in CPLX else 0.5
    Xb = orc.solve_batched(L, B, a)
    for p in range(5):
        assert bits_equal(np.asfortranarray(Xb[p]), orc.solve(L[p], B[p], a)), (dtype, p)


VARIANTS = [(s, u, t, d) for s in "LR" for u in "LU" for t in "NTC" for d in "NU"]


def _variant_problem(dtype, side, uplo, diag, m, n, seed):
    """A with the unused triangle (and, for a unit diagonal, the diagonal)
    set to NaN: the solve must not read them."""
    rng = np.random.default_rng(seed)
    k = m if side == "L" else n
    A = rng.uniform(-1, 1, (k, k)) / k + np.diag(rng.uniform(1, 2, k))
    if dtype in CPLX:
        A = A + 1j * rng.uniform(-1, 1, (k, k)) / k
    B = rng.uniform(-1, 1, (m, n)) + (1j * rng.uniform(-1, 1, (m, n)) if dtype in CPLX else 0)
    clean = np.asfortranarray(A.astype(NP[dtype]))
    poisoned = clean.copy()
    bad = np.triu(np.ones((k, k), bool), 1) if uplo == "L" else np.tril(np.ones((k, k), bool), -1)
    if diag == "U":
        bad |= np.eye(k, dtype=bool)
    poisoned[bad] = np.nan
    return clean, np.asfortranarray(poisoned), np.asfortranarray(B.astype(NP[dtype]))


def check_variants_scipy(orc, dtype):
    """Every (side, uplo, trans, diag) against scipy's BLAS ?trsm (for real
    data trans 'C' is 'T'), with the entries that must not be read set to NaN
    in the oracle's input."""
    tol = {"f32": 5e-6, "f64": 1e-14, "c64": 1e-14, "c32": 5e-6}[dtype]
    trsm = {"f32": sblas.strsm, "f64": sblas.dtrsm, "c64": sblas.ztrsm, "c32": sblas.ctrsm}[dtype]
    a = 0.75 - 0.25j if dtype in CPLX else -0.75
    for idx, (side, uplo, trans, diag) in enumerate(VARIANTS):
        m, n = (13, 7) if idx % 2 else (6, 11)
        clean, poisoned, B = _variant_problem(dtype, side, uplo, diag, m, n, seed=idx)
        X = orc.trsm(side, uplo, trans, diag, poisoned, B, a)
        t = {"N": 0, "T": 1, "C": 2 if dtype in CPLX else 1}[trans]
        ref = trsm(a, np.array(clean, order="F"), np.array(B, order="F"), side=int(side == "R"),
                   lower=int(uplo == "L"), trans_a=t, diag=int(diag == "U"))
        assert np.all(np.isfinite(X)), (dtype, side, uplo, trans, diag)
        assert nrel(X, ref) < tol, (dtype, side, uplo, trans, diag, nrel(X, ref))


QUICK_CHECKS = [check_identity, check_diagonal, check_bidiagonal, check_exact_dyadic,
                check_scipy, check_batched_matches_single, check_variants_scipy]


# ---------------------------------------------------------------------------
# tests on the real oracle
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def orc():
    return oracle._load()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("check", QUICK_CHECKS, ids=lambda f: f.__name__)
def test_quick_pins(orc, check, dtype):
    check(orc, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_force_non_dyadic(orc, dtype):
    """Integer systems with diagonals 3, 5, -3, 7: the oracle must sit within
    a few ulp (normwise) of the exact solution from Gauss-Jordan."""
    rng = np.random.default_rng(5)
    u = UNIT_ROUNDOFF[dtype]
    for trial in range(15):
        m = int(rng.integers(1, 7))
        n = int(rng.integers(1, 5))
        L = random_integer_lower(m, dtype, rng, [3.0, 5.0, -3.0, 7.0, 1.0])
        B = small_integer_rhs(m, n, dtype, seed=100 + trial)
        a = 0.75 - 0.5j if dtype in CPLX else 0.75
        X = orc.solve(L, B, a)
        Xe = exact_solution(L, B, a)
        assert nrel(X, Xe) <= 8 * m * u, (dtype, trial, nrel(X, Xe))


def test_loop_order_invariance(orc):
    """Column ("axpy") order == row-wise dot order, bitwise; each column
    solved alone == the same column solved with the others, bitwise."""
    for m, n in [(1, 1), (5, 300), (300, 17), (129, 64)]:
        L, B = make_problem("f64", m, n, seed=m + n)
        for a in [1.0, 0.3]:
            Xc = orc.solve(L, B, a)
            Xr = orc.solve(L, B, a, rowdot=True)
            assert bits_equal(Xc, Xr), (m, n, a)
            for j in sorted({0, n // 2, n - 1}):
                xj = orc.solve(L, np.asfortranarray(B[:, j:j + 1]), a)
                assert bits_equal(xj[:, 0], Xc[:, j])


@pytest.mark.parametrize("dtype", DTYPES)
def test_variant_oracle_left_lower_is_the_pinned_solve(orc, dtype):
    """The general oracle at (side L, lower, no transpose, non-unit) runs the
    same operations in the same order as the pinned left-lower solve:
    bitwise equal."""
    for m, n in [(1, 1), (64, 64), (150, 37)]:
        L, B = make_problem(dtype, m, n, seed=m + 2 * n)
        a = 0.5 - 0.25j if dtype in CPLX else 0.5
        assert bits_equal(orc.trsm("L", "L", "N", "N", L, B, a), orc.solve(L, B, a)), (dtype, m, n)


@pytest.mark.parametrize("dtype", DTYPES)
def test_alpha_scaling(orc, dtype):
    L, B = make_problem(dtype, 80, 10, seed=8)
    a = 0.3 + 0.2j if dtype in CPLX else 0.3
    X1 = orc.solve(L, B, 1.0)
    Xa = orc.solve(L, B, a)
    assert nrel(Xa, np.asarray(a) * X1) < 20 * UNIT_ROUNDOFF[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
def test_alpha_zero_does_not_read_A(orc, dtype):
    m, n = 9, 4
    L = np.full((m, m), np.nan, dtype=NP[dtype], order="F")
    _, B = make_problem(dtype, m, n, seed=1)
    X = orc.solve(L, B, 0.0)
    assert np.all(X == 0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_upper_triangle_and_padding_not_read(orc, dtype):
    L0, B0 = make_problem(dtype, 70, 9, seed=4)
    Ln, Bp = make_problem(dtype, 70, 9, seed=4, lda=77, ldb=81, upper="nan")
    X0 = orc.solve(L0, B0, 0.5)
    Xn = orc.solve(Ln, Bp, 0.5)
    assert bits_equal(X0, Xn)


@pytest.mark.parametrize("dtype", DTYPES)
def test_residual_bound_configs(orc, dtype):
    """Backward stability: ||L X - alpha B|| / (||L|| ||X|| + |alpha| ||B||)
    stays below c*m*u on every workload of this dtype (large ones on a few
    sampled right-hand-side columns at full m; columns are independent)."""
    u = UNIT_ROUNDOFF[dtype]
    for cfg in CONFIGS.values():
        if cfg.dtype != dtype:
            continue
        L, B, a = make_config(cfg)
        if cfg.batch:
            L, B = L[:16], B[:16]
            X = orc.solve_batched(L, B, a)
            pairs = [(L[p], B[p], X[p]) for p in range(16)]
        else:
            cols = np.unique(np.linspace(0, cfg.n - 1, 4).astype(int)) if cfg.m > 64 else slice(None)
            Bs = np.asfortranarray(B[:, cols])
            pairs = [(L, Bs, orc.solve(L, Bs, a))]
        for Lp, Bp, Xp in pairs:
            Lw = np.asarray(Lp, dtype=np.complex128)
            R = Lw @ np.asarray(Xp, dtype=np.complex128) - a * np.asarray(Bp, dtype=np.complex128)
            den = np.linalg.norm(Lw) * np.linalg.norm(Xp) + abs(a) * np.linalg.norm(Bp)
            assert np.linalg.norm(R) / den <= 10 * cfg.m * u, (cfg.name, np.linalg.norm(R) / den)


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_error_scale_vs_pages_table2(orc, dtype):
    """Against an independent TRSM (scipy/LAPACK) at m = n = 1024 the oracle's
    normwise difference is of the order the pages report against a vendor
    TRSM (Table 2), i.e. at most 10x that figure."""
    table = json.load(open(os.path.join(HERE, "golden", "table2_normwise_error.json")))
    ref_err = table["error"][dtype][table["sizes"].index(1024)]
    m = n = 1024
    L, B = make_problem(dtype, m, n, seed=1024)
    X = orc.solve(L, B, 1.0)
    ref = sla.solve_triangular(np.array(L), np.array(B), lower=True)
    e = nrel(X, ref)
    assert e <= 10 * ref_err, (dtype, e, ref_err)


# ---------------------------------------------------------------------------
# planted mistakes: every mutant of the oracle must fail a quick pin
# ---------------------------------------------------------------------------

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle_lln.c")

# (name, function body to mutate, old text, new text)
MUTANTS = [
    ("f64_sign", "solve_column_d", "b[i] = b[i] - lk[i] * xk;", "b[i] = b[i] + lk[i] * xk;"),
    ("f64_transposed", "solve_column_d", "b[i] = b[i] - lk[i] * xk;",
     "b[i] = b[i] - A[k + i * lda] * xk;"),
    ("f64_dropped_alpha", "solve_column_d", "b[i] = alpha * b[i];", "b[i] = b[i];"),
    ("f64_dropped_term", "solve_column_d", "for (i = k + 1; i < m; ++i)",
     "for (i = k + 2; i < m; ++i)"),
    ("f64_no_divide", "solve_column_d", "double xk = b[k] / lk[k];", "double xk = b[k];"),
    ("f64_wrong_pivot", "solve_column_d", "double xk = b[k] / lk[k];",
     "double xk = b[k] / lk[k > 0 ? k - 1 : 0];"),
    ("f32_sign", "solve_column_s", "b[i] = b[i] - lk[i] * xk;", "b[i] = b[i] + lk[i] * xk;"),
    ("f32_transposed", "solve_column_s", "b[i] = b[i] - lk[i] * xk;",
     "b[i] = b[i] - A[k + i * lda] * xk;"),
    ("z_conj_product_re", "solve_column_z", "double pr = lr * xr - li * xi;",
     "double pr = lr * xr + li * xi;"),
    ("z_conj_product_im", "solve_column_z", "double pi = lr * xi + li * xr;",
     "double pi = lr * xi - li * xr;"),
    ("z_alpha_sign", "solve_column_z", "b[2 * i]     = ar * br - ai * bi;",
     "b[2 * i]     = ar * br + ai * bi;"),
    ("z_div_sign", "solve_column_z", "xi = (bi * dr - br * di) / den;",
     "xi = (bi * dr + br * di) / den;"),
    ("z_real_div", "solve_column_z", "xi = bi / dr;", "xi = bi * dr;"),
    ("z_swapped_parts", "solve_column_z", "double lr = lk[2 * i], li = lk[2 * i + 1];",
     "double li = lk[2 * i], lr = lk[2 * i + 1];"),
    ("c_conj_product_im", "solve_column_c", "float pi = lr * xi + li * xr;",
     "float pi = lr * xi - li * xr;"),
    ("c_div_sign", "solve_column_c", "xi = (bi * dr - br * di) / den;",
     "xi = (bi * dr + br * di) / den;"),
    ("c_swapped_parts", "solve_column_c", "float lr = lk[2 * i], li = lk[2 * i + 1];",
     "float li = lk[2 * i], lr = lk[2 * i + 1];"),
    ("c_alpha_dropped_im", "solve_column_c", "b[2 * i + 1] = ar * bi + ai * br;",
     "b[2 * i + 1] = ar * bi;"),
    ("c_batched_stride", "oracle_lln_c_batched", "solve_column_c(m, alpha_re, alpha_im, A + 2 * p * strideA, lda,",
     "solve_column_c(m, alpha_re, alpha_im, A + p * strideA, lda,"),
    ("trsm_right_untransposed", "tget_d", "if (side == 1) { r = k; c = i; }", "if (side == 1) { r = i; c = k; }"),
    ("trsm_no_conj", "tget_d", "if (trans == 2) *im = -*im;", "if (trans == 3) *im = -*im;"),
    ("trsm_wrong_triangle", "oracle_trsm_d", "int op_lower = (uplo == 0) == (trans == 0);",
     "int op_lower = (uplo == 0);"),
    ("trsm_unit_divides", "oracle_trsm_d", "if (!diag) {", "if (1) {"),
    ("trsm_s_alpha_im_sign", "oracle_trsm_s", "float si = alpha_re * ci + alpha_im * cr;",
     "float si = alpha_re * ci - alpha_im * cr;"),
    ("batched_stride", "oracle_lln_d_batched", "solve_column_d(m, alpha, A + p * strideA, lda,",
     "solve_column_d(m, alpha, A, lda,"),
]


def _mutate(src, func, old, new):
    start = src.index(func + "(")
    # the body of `func` starts at its definition; mutate the first match after it
    pos = src.index(old, start)
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_mistakes_are_caught():
    src = open(SRC).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    survivors = []
    try:
        for name, func, old, new in MUTANTS:
            msrc = _mutate(src, func, old, new)
            assert msrc != src
            c = os.path.join(tmp, f"{name}.c")
            so = os.path.join(tmp, f"lib{name}.so")
            open(c, "w").write(msrc)
            subprocess.run(["gcc", *oracle.CFLAGS, c, "-o", so], check=True)
            mut = oracle.OracleLib(so)
            caught = False
            for check in QUICK_CHECKS:
                for dtype in DTYPES:
                    try:
                        with np.errstate(all="ignore"):
                            check(mut, dtype)
                    except (AssertionError, StopIteration, ZeroDivisionError, ValueError):
                        caught = True
                        break
                if caught:
                    break
            if not caught:
                survivors.append(name)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    assert not survivors, f"mutants not caught by any pin: {survivors}"
