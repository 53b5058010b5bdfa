"""CPU oracle for left-lower TRSM (L X = alpha B), loaded through ctypes.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.

The arithmetic lives in ``oracle_lln.c`` (plain C, -O2 -ffp-contract=off,
OpenMP over independent columns / batch entries).  It follows the
forward-substitution formula of HSMA-TRSM ("Hierarchical Shared Memory-Aware
Optimization for TRSM on GPU Platforms", section 2.1 and the equation of
section 4.2.1).  This module only marshals numpy arrays.

Every function here is pinned by tests that do not re-type the formula:
identity and diagonal L (bitwise), the unit bidiagonal L with -1 below the
diagonal whose inverse is the all-ones lower triangle (bitwise), exact
rational brute force on tiny systems, the residual bound, loop-order
invariance, and agreement with scipy's LAPACK/BLAS triangular solve.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_lln.c")
_LIB = os.path.join(_HERE, "liboracle_lln.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile oracle_lln.c into liboracle_lln.so with gcc (host only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class OracleLib:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, dbl, flt, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_float, ctypes.c_void_p
        lib.oracle_lln_d.argtypes = [i64, i64, dbl, vp, i64, vp, i64]
        lib.oracle_lln_d_rowdot.argtypes = [i64, i64, dbl, vp, i64, vp, i64]
        lib.oracle_lln_s.argtypes = [i64, i64, flt, vp, i64, vp, i64]
        lib.oracle_lln_z.argtypes = [i64, i64, dbl, dbl, vp, i64, vp, i64]
        lib.oracle_lln_d_batched.argtypes = [i64, i64, dbl, vp, i64, i64, vp, i64, i64, i64]
        lib.oracle_lln_s_batched.argtypes = [i64, i64, flt, vp, i64, i64, vp, i64, i64, i64]
        lib.oracle_lln_z_batched.argtypes = [i64, i64, dbl, dbl, vp, i64, i64, vp, i64, i64, i64]
        lib.oracle_lln_c.argtypes = [i64, i64, flt, flt, vp, i64, vp, i64]
        lib.oracle_lln_c_batched.argtypes = [i64, i64, flt, flt, vp, i64, i64, vp, i64, i64, i64]
        ci = ctypes.c_int
        lib.oracle_trsm_d.argtypes = [ci, ci, ci, ci, ci, i64, i64, dbl, dbl, vp, i64, vp, i64]
        lib.oracle_trsm_s.argtypes = [ci, ci, ci, ci, ci, i64, i64, flt, flt, vp, i64, vp, i64]
        for f in ("oracle_lln_d", "oracle_lln_d_rowdot", "oracle_lln_s", "oracle_lln_z",
                  "oracle_lln_c", "oracle_lln_d_batched", "oracle_lln_s_batched",
                  "oracle_lln_z_batched", "oracle_lln_c_batched", "oracle_trsm_d",
                  "oracle_trsm_s"):
            getattr(lib, f).restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def solve(self, L: np.ndarray, B: np.ndarray, alpha=1.0, *, rowdot: bool = False) -> np.ndarray:
        """Return X with L X = alpha B (a copy of B solved in place).

        L: m x m, B: m x n, column-major (or any layout: copied to Fortran
        order), dtype float32, float64, complex64 or complex128.  Only the lower
        triangle of L is read."""
        m = L.shape[0]
        if L.shape != (m, m) or B.shape[0] != m or L.dtype != B.dtype:
            raise ValueError("shape/dtype mismatch")
        X = np.array(B, order="F", copy=True)
        n = X.shape[1]
        lib = self.lib
        L, lda = _colmajor(L)
        ldx = max(m, 1)
        if L.dtype == np.float64:
            f = lib.oracle_lln_d_rowdot if rowdot else lib.oracle_lln_d
            rc = f(m, n, float(alpha), L.ctypes.data, lda, X.ctypes.data, ldx)
        elif rowdot:
            raise ValueError("the row-wise dot form exists for float64 only")
        elif L.dtype == np.float32:
            rc = lib.oracle_lln_s(m, n, float(alpha), L.ctypes.data, lda, X.ctypes.data, ldx)
        elif L.dtype == np.complex128:
            a = complex(alpha)
            rc = lib.oracle_lln_z(m, n, a.real, a.imag, L.ctypes.data, lda, X.ctypes.data, ldx)
        elif L.dtype == np.complex64:
            a = complex(alpha)
            rc = lib.oracle_lln_c(m, n, a.real, a.imag, L.ctypes.data, lda, X.ctypes.data, ldx)
        else:
            raise TypeError(f"unsupported dtype {L.dtype}")
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return X

    def solve_batched(self, L: np.ndarray, B: np.ndarray, alpha=1.0) -> np.ndarray:
        """Batched solve.  L: (batch, m, m), B: (batch, m, n), each problem
        column-major.  Returns X with the shape of B (a new array)."""
        batch, m, _ = L.shape
        n = B.shape[2]
        # canonical storage: per problem column-major, problems contiguous
        Lc = np.ascontiguousarray(np.transpose(L, (0, 2, 1)))
        Xc = np.array(np.transpose(B, (0, 2, 1)), order="C", copy=True)
        lib = self.lib
        sA, sB, ld = m * m, m * n, max(m, 1)
        if L.dtype == np.float64:
            rc = lib.oracle_lln_d_batched(m, n, float(alpha), Lc.ctypes.data, ld, sA,
                                          Xc.ctypes.data, ld, sB, batch)
        elif L.dtype == np.float32:
            rc = lib.oracle_lln_s_batched(m, n, float(alpha), Lc.ctypes.data, ld, sA,
                                          Xc.ctypes.data, ld, sB, batch)
        elif L.dtype == np.complex128:
            a = complex(alpha)
            rc = lib.oracle_lln_z_batched(m, n, a.real, a.imag, Lc.ctypes.data, ld, sA,
                                          Xc.ctypes.data, ld, sB, batch)
        elif L.dtype == np.complex64:
            a = complex(alpha)
            rc = lib.oracle_lln_c_batched(m, n, a.real, a.imag, Lc.ctypes.data, ld, sA,
                                          Xc.ctypes.data, ld, sB, batch)
        else:
            raise TypeError(f"unsupported dtype {L.dtype}")
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return np.transpose(Xc, (0, 2, 1))


    def trsm(self, side: str, uplo: str, trans: str, diag: str, A: np.ndarray, B: np.ndarray,
             alpha=1.0) -> np.ndarray:
        """General TRSM by its definition: op(A) X = alpha B (side 'L', A
        m x m) or X op(A) = alpha B (side 'R', A n x n); uplo 'L'/'U' names
        the triangle of A that is used, trans 'N'/'T'/'C' gives op(A) = A,
        A^T or A^H, diag 'N'/'U' non-unit or unit (then the diagonal of A is
        not read).  Returns X (a new array)."""
        codes = ({"L": 0, "R": 1}[side], {"L": 0, "U": 1}[uplo], {"N": 0, "T": 1, "C": 2}[trans],
                 {"N": 0, "U": 1}[diag])
        m, n = B.shape
        k = m if side == "L" else n
        if A.shape != (k, k) or A.dtype != B.dtype:
            raise ValueError("shape/dtype mismatch")
        X = np.array(B, order="F", copy=True)
        A, lda = _colmajor(A)
        cplx = int(np.iscomplexobj(A))
        a = complex(alpha)
        if A.dtype in (np.float64, np.complex128):
            f = self.lib.oracle_trsm_d
        elif A.dtype in (np.float32, np.complex64):
            f = self.lib.oracle_trsm_s
        else:
            raise TypeError(f"unsupported dtype {A.dtype}")
        rc = f(*codes, cplx, m, n, a.real, a.imag, A.ctypes.data, lda, X.ctypes.data, max(m, 1))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return X


_default = None


def _load() -> OracleLib:
    global _default
    if _default is None:
        _default = OracleLib(build())
    return _default


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use (OMP_NUM_THREADS)."""
    return _load().num_threads()


def solve(L, B, alpha=1.0, *, rowdot: bool = False):
    """Module-level shortcut for OracleLib.solve on the default build."""
    return _load().solve(L, B, alpha, rowdot=rowdot)


def trsm(side, uplo, trans, diag, A, B, alpha=1.0):
    return _load().trsm(side, uplo, trans, diag, A, B, alpha)


def solve_batched(L, B, alpha=1.0):
    """Module-level shortcut for OracleLib.solve_batched on the default build."""
    return _load().solve_batched(L, B, alpha)


def _colmajor(a: np.ndarray):
    """(array, leading dimension) of a 2-D operand in column-major storage.

    Fortran-contiguous arrays and column-major views of a padded buffer
    (strides (itemsize, ld*itemsize), ld >= rows) pass through unchanged;
    anything else is copied to Fortran order."""
    if a.ndim != 2:
        raise ValueError("expected a 2-D array")
    item = a.itemsize
    rows, cols = a.shape
    unit_rows = rows <= 1 or a.strides[0] == item
    if unit_rows and cols > 1 and a.strides[1] % item == 0 and a.strides[1] // item >= max(rows, 1):
        return a, a.strides[1] // item
    if unit_rows and cols <= 1:
        return a, max(rows, 1)
    a = np.asfortranarray(a)
    return a, max(rows, 1)
