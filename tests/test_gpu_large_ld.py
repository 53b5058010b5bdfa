"""Parity at leading dimensions too large for 32-bit offsets inside a tile.

The BLAS rules (HSMA-TRSM section 2.1's system, column-major operands with
lda, ldb >= m) allow a small problem to sit in a huge array: a sub-block
of a tall matrix has an ldb of millions.  The GEMMs read a tile of up to 128
columns through 32-bit buffer offsets, and the inversion a diagonal block of
64 columns; past 2 GB of such a span they switch to 64-bit addressing.  Each
case here puts lda or ldb past that point on the blocked path (and, for the
direct path, past the 2 GB range of one problem), compares with the oracle,
and checks that B's rows past m are untouched.

Operands are built on the device (a padded buffer filled on the GPU, the
m x n values copied in), so the host only holds the m x n problem.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import CPLX, TOL, nrel, torch_dtype
from trsm_inputs import make_problem

pytestmark = pytest.mark.gpu

ESIZE = {"f32": 4, "f64": 8, "c64": 16, "c32": 8}


def wide_ld(dtype, cols):
    """Smallest leading dimension whose `cols` columns span 2 GB or more."""
    return (2 ** 31) // (ESIZE[dtype] * cols) + 17


def padded_on_device(a, ld, pad):
    """(view, base): base is an n x ld device buffer filled with `pad`; view
    is its first m rows as an m x n column-major operand holding `a`."""
    import torch
    m, n = a.shape
    base = torch.full((n, ld), pad, dtype=torch_dtype_of(a), device="cuda")
    base[:, :m] = torch.from_numpy(np.ascontiguousarray(a.T)).cuda()
    return base.T[:m], base


def torch_dtype_of(a):
    import torch
    return {np.float32: torch.float32, np.float64: torch.float64, np.complex64: torch.complex64,
            np.complex128: torch.complex128}[a.dtype.type]


def pad_value(dtype, v):
    return complex(v, v) if dtype in CPLX else v


CASES = [
    # (dtype, m, n, lda, ldb): ldb past the widest GEMM tile's 2 GB span
    ("f64", 1000, 8, 1000, 2_200_000),
    ("c64", 300, 8, 300, 1_100_000),
    ("f32", 700, 5, 700, wide_ld("f32", 128)),
    ("c32", 500, 6, 500, wide_ld("c32", 128)),
    # lda past the inversion's 64-column span (fp64: 4.3 M)
    ("f64", 100, 9, 4_300_000, 100),
    # lda past the GEMM's A tile span too (32 columns), ldb past 8 columns
    ("f64", 130, 3, wide_ld("f64", 32), wide_ld("f64", 8)),
    ("c64", 90, 4, wide_ld("c64", 32), 90),
    ("f32", 150, 7, wide_ld("f32", 32), 150),
    ("c32", 110, 5, wide_ld("c32", 32), wide_ld("c32", 128)),
    # direct path (m <= 64): one problem spans more than 2 GB
    ("f64", 50, 70, wide_ld("f64", 49), wide_ld("f64", 69)),
    ("c64", 64, 3, 64, wide_ld("c64", 2)),
    ("f32", 40, 66, wide_ld("f32", 39), 40),
    ("c32", 33, 2, 33, wide_ld("c32", 1)),
]


@pytest.mark.parametrize("dtype,m,n,lda,ldb", CASES)
def test_large_leading_dimensions(dtype, m, n, lda, ldb):
    import torch
    import triangular_solve_trsm_amd as T
    print(f"case {dtype} m={m} n={n} lda={lda} ldb={ldb}", flush=True)
    L, B = make_problem(dtype, m, n, seed=m + n)
    a = 0.75 - 0.5j if dtype in CPLX else 0.75
    Ad, Abase = padded_on_device(L, lda, pad_value(dtype, float("nan")))
    Bd, Bbase = padded_on_device(B, ldb, pad_value(dtype, 777.0))
    T.trsm_lln(Ad, Bd, a)
    torch.cuda.synchronize()
    # rows past m of every column of B are untouched
    tail = Bbase[:, m:]
    assert bool(torch.all(tail == pad_value(dtype, 777.0)).item()), "B's rows past m were modified"
    X = Bd.cpu().numpy()
    del Abase, Bbase, Ad, Bd, tail
    torch.cuda.empty_cache()
    e = nrel(X, oracle.solve(L, B, a))
    assert e <= TOL[dtype] and e <= TOL[dtype] / 10, (dtype, m, n, lda, ldb, e)
