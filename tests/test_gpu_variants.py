"""GPU parity of the general TRSM (trsm_solve) against the oracle's
definition-level solve, for every side, triangle, transposition and
diagonal in every data type.

Every variant is solved by the library as a left-lower solve after an index
reflection of A (and of B when the right-hand sides must be reordered); the
oracle solves each right-hand side by substitution in the direction its
triangle allows, with no reflection.  The entries the solve must not read
(the other triangle of A, and its diagonal when the diagonal is unit) are NaN
on the device.  Sizes cover the direct path (order <= 64) and the blocked
path with ragged blocks.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import CPLX, NP, TOL, from_dev, nrel, to_dev

pytestmark = pytest.mark.gpu

VARIANTS = [(s, u, t, d) for s in "LR" for u in "LU" for t in "NTC" for d in "NU"]


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import triangular_solve_trsm_amd as T
    return T


def problem(dtype, side, uplo, diag, m, n, seed):
    rng = np.random.default_rng(seed)
    k = m if side == "L" else n
    A = rng.uniform(-1, 1, (k, k)) / k + np.diag(rng.uniform(1, 2, k))
    B = rng.uniform(-1, 1, (m, n))
    if dtype in CPLX:
        A = A + 1j * rng.uniform(-1, 1, (k, k)) / k
        B = B + 1j * rng.uniform(-1, 1, (m, n))
    A = np.asfortranarray(A.astype(NP[dtype]))
    bad = np.triu(np.ones((k, k), bool), 1) if uplo == "L" else np.tril(np.ones((k, k), bool), -1)
    if diag == "U":
        bad |= np.eye(k, dtype=bool)
    A[bad] = np.nan
    return A, np.asfortranarray(B.astype(NP[dtype]))


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("m,n", [(50, 37), (300, 130), (129, 700)])
def test_every_variant(T, dtype, m, n):
    import torch
    a = 0.75 - 0.5j if dtype in CPLX else -0.75
    worst = 0.0
    for idx, (side, uplo, trans, diag) in enumerate(VARIANTS):
        A, B = problem(dtype, side, uplo, diag, m, n, seed=1000 * idx + m + n)
        Ad, Bd = to_dev(A, ld=A.shape[0] + 3), to_dev(B, ld=m + 2, pad=777.0)
        T.trsm_solve(Ad, Bd, a, side=side, uplo=uplo, trans=trans, diag=diag)
        torch.cuda.synchronize()
        X = from_dev(Bd)
        ref = oracle.trsm(side, uplo, trans, diag, A, B, a)
        e = nrel(X, ref)
        assert np.all(np.isfinite(X)), (dtype, side, uplo, trans, diag, "non-finite: a NaN entry was read")
        assert e <= TOL[dtype], (dtype, m, n, side, uplo, trans, diag, e)
        worst = max(worst, e)
        full = from_dev(torch.as_strided(Bd, (m + 2, n), (1, m + 2)))
        assert np.all(full[m:] == 777.0), "padding rows of B were modified"
    print(f"{dtype} {m}x{n}: worst error over the 24 variants {worst:.2e}")


@pytest.mark.parametrize("dtype", ["f64", "c64"])
def test_left_lower_is_trsm_lln(T, dtype):
    """trsm_solve(L, L, N, N) is the left-lower solve itself: bitwise equal."""
    import torch
    from trsm_inputs import make_problem
    L, B = make_problem(dtype, 400, 90, seed=4)
    B1, B2 = to_dev(B), to_dev(B)
    T.trsm_lln(to_dev(L), B1, 0.5)
    T.trsm_solve(to_dev(L), B2, 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(B1), from_dev(B2))


def test_alpha_zero_does_not_read_A(T):
    import torch
    from trsm_inputs import make_problem
    _, B = make_problem("c64", 70, 20, seed=3)
    Bd = to_dev(B)
    Ad = to_dev(np.full((20, 20), np.nan, dtype=np.complex128, order="F"))
    T.trsm_solve(Ad, Bd, 0.0, side="R", uplo="U", trans="C", diag="U")
    torch.cuda.synchronize()
    assert torch.all(Bd == 0).item()
