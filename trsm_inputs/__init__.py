"""Seeded synthetic inputs for left-lower TRSM (L X = alpha B).

This module is shared by the tests, the benchmark and the smoke check.  It
holds only input recipes (random draws, layouts, special matrices); it does no
part of the solve.  Neither the oracle nor the HIP library imports it.

Recipe (the pages evaluate on random inputs and do not give a distribution;
HSMA-TRSM, section 5.1 "Test Configuration"):

* generator ``numpy.random.default_rng(seed)`` (PCG64);
* real L: ``U = rng.uniform(-1, 1, (m, m))``, ``d = rng.uniform(1, 2, m)``;
  ``L[i, k] = U[i, k] / m`` for i > k, ``L[i, i] = d[i]``, zero above the
  diagonal; then ``B = rng.uniform(-1, 1, (m, n))``;
* complex L: the real part of U, then its imaginary part, then d (real
  diagonal, imaginary part 0), then the real and imaginary parts of B;
* batched problems: the same draws with a leading batch axis on every array,
  whole arrays drawn in the order above;
* fp32 and complex-fp32 problems are drawn in float64 and rounded to
  float32 parts;
* storage is column-major per problem (element (i, j) at ``i + j*ld``).

Off-diagonal magnitudes of at most 1/m (sqrt(2)/m for complex) against a
diagonal in [1, 2] make every L strictly row-diagonally dominant, hence well
conditioned, so the normwise error of a correct solve sits near the unit
roundoff times a modest factor.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

SEED_BASE = 20261201

_NP_DTYPE = {"f32": np.float32, "f64": np.float64, "c64": np.complex128, "c32": np.complex64}
_COMPLEX = ("c64", "c32")


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str          # "f32" | "f64" | "c64" | "c32"  (complex fp64 / fp32)
    m: int
    n: int
    alpha: complex
    batch: Optional[int]  # None for a single problem
    index: int            # 1-based position in the workload list (seed offset)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def flops(self) -> float:
        """Counted flops: m^2 n (real), 4 m^2 n (complex), per problem times batch."""
        f = float(self.m) * self.m * self.n * (4.0 if self.dtype in _COMPLEX else 1.0)
        return f * (self.batch or 1)


# The five workloads: one small fp64 solve, a batch of small complex solves,
# and three large solves of the blocked regime.
CONFIGS = {
    "c1_f64_64": Config("c1_f64_64", "f64", 64, 64, 1.0, None, 1),
    "c2_c64_64x64_b8192": Config("c2_c64_64x64_b8192", "c64", 64, 64, 1.0 + 0j, 8192, 2),
    "c3_f32_4096": Config("c3_f32_4096", "f32", 4096, 4096, 0.5, None, 3),
    "c4_f64_8192": Config("c4_f64_8192", "f64", 8192, 8192, 1.0, None, 4),
    "c5_c64_8192x2048": Config("c5_c64_8192x2048", "c64", 8192, 2048, 1.0 + 0j, None, 5),
}


def np_dtype(dtype: str):
    return _NP_DTYPE[dtype]


def _colmajor_empty(rows: int, cols: int, ld: int, dtype, batch: Optional[int], fill):
    """Column-major storage (per problem) with leading dimension ld >= rows.

    Returns (view, base): view has shape (rows, cols) or (batch, rows, cols);
    rows beyond `rows` in each column hold `fill`."""
    if batch is None:
        base = np.full((cols, ld), fill, dtype=dtype)
        return base.T[:rows, :], base
    base = np.full((batch, cols, ld), fill, dtype=dtype)
    return np.transpose(base, (0, 2, 1))[:, :rows, :], base


def make_problem(dtype: str, m: int, n: int, seed: int, *, batch: Optional[int] = None,
                 lda: Optional[int] = None, ldb: Optional[int] = None,
                 upper: str = "zero", pad_fill=np.nan):
    """Draw (L, B) by the recipe above.

    Returns column-major numpy views: L (m, m) and B (m, n), or with a leading
    batch axis.  ``upper='nan'`` fills the strict upper triangle of L with NaN
    (it must never be read); padding rows (lda > m, ldb > m) hold ``pad_fill``.
    """
    if dtype not in _NP_DTYPE:
        raise ValueError(f"unknown dtype {dtype}")
    lda = max(m, 1) if lda is None else lda
    ldb = max(m, 1) if ldb is None else ldb
    rng = np.random.default_rng(seed)
    shp_u = (m, m) if batch is None else (batch, m, m)
    shp_d = (m,) if batch is None else (batch, m)
    shp_b = (m, n) if batch is None else (batch, m, n)
    if dtype in _COMPLEX:
        U = rng.uniform(-1.0, 1.0, shp_u) + 1j * rng.uniform(-1.0, 1.0, shp_u)
        d = rng.uniform(1.0, 2.0, shp_d).astype(np.complex128)
        Bv = rng.uniform(-1.0, 1.0, shp_b) + 1j * rng.uniform(-1.0, 1.0, shp_b)
    else:
        U = rng.uniform(-1.0, 1.0, shp_u)
        d = rng.uniform(1.0, 2.0, shp_d)
        Bv = rng.uniform(-1.0, 1.0, shp_b)
    npd = _NP_DTYPE[dtype]
    Lfull = np.tril(U, -1) / m
    idx = np.arange(m)
    Lfull[..., idx, idx] = d
    if upper == "nan":
        iu = np.triu_indices(m, 1)
        Lfull[..., iu[0], iu[1]] = np.nan
    elif upper != "zero":
        raise ValueError("upper must be 'zero' or 'nan'")
    L, _ = _colmajor_empty(m, m, lda, npd, batch, pad_fill)
    L[...] = Lfull.astype(npd)
    B, _ = _colmajor_empty(m, n, ldb, npd, batch, pad_fill)
    B[...] = Bv.astype(npd)
    return L, B


def make_config(cfg: Config, **kw):
    """(L, B, alpha) for one of CONFIGS, drawn with the config's seed."""
    L, B = make_problem(cfg.dtype, cfg.m, cfg.n, cfg.seed, batch=cfg.batch, **kw)
    alpha = complex(cfg.alpha) if cfg.dtype in _COMPLEX else float(np.real(cfg.alpha))
    return L, B, alpha


# ---- structured inputs with known solutions (used as pins) -----------------

def identity(m: int, dtype: str):
    return np.asfortranarray(np.eye(m, dtype=_NP_DTYPE[dtype]))


def diagonal(diag: np.ndarray, dtype: str):
    return np.asfortranarray(np.diag(np.asarray(diag)).astype(_NP_DTYPE[dtype]))


def unit_bidiagonal_minus_one(m: int, dtype: str):
    """Ones on the diagonal, -1 on the first sub-diagonal, zero elsewhere."""
    L = np.eye(m, dtype=_NP_DTYPE[dtype])
    if m > 1:
        L[np.arange(1, m), np.arange(m - 1)] = -1
    return np.asfortranarray(L)


def small_integer_rhs(m: int, n: int, dtype: str, seed: int, lo: int = -8, hi: int = 8):
    """Integer-valued B (real and imaginary parts for complex) in [lo, hi]."""
    rng = np.random.default_rng(seed)
    if dtype in _COMPLEX:
        B = rng.integers(lo, hi + 1, (m, n)) + 1j * rng.integers(lo, hi + 1, (m, n))
    else:
        B = rng.integers(lo, hi + 1, (m, n))
    return np.asfortranarray(B.astype(_NP_DTYPE[dtype]))
