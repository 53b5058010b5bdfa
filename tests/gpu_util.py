"""Helpers for GPU tests: move column-major numpy operands to the device
keeping their leading dimension, call the library through its binding, and
measure normwise errors."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "f64": 1e-12, "c64": 1e-12, "c32": 1e-4}   # normwise relative error vs the oracle
NP = {"f32": np.float32, "f64": np.float64, "c64": np.complex128, "c32": np.complex64}
CPLX = ("c64", "c32")


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f64": torch.float64, "c64": torch.complex128,
            "c32": torch.complex64}[dtype]


def ld_of(a):
    """Leading dimension of a column-major numpy view (2-D or batched 3-D)."""
    item = a.itemsize
    if a.ndim == 2:
        return a.strides[1] // item if a.shape[1] > 1 else max(a.shape[0], 1)
    return a.strides[2] // item if a.shape[2] > 1 else max(a.shape[1], 1)


def to_dev(a, *, ld=None, pad=np.nan, device="cuda"):
    """Column-major device copy of `a` with leading dimension ld (default:
    that of `a`); padding rows hold `pad`."""
    import torch
    ld = ld_of(a) if ld is None else ld
    if a.ndim == 2:
        m, n = a.shape
        base = np.full((n, ld), pad, dtype=a.dtype)
        base.T[:m] = a
        return torch.from_numpy(base).to(device).T[:m]
    b, m, n = a.shape
    base = np.full((b, n, ld), pad, dtype=a.dtype)
    np.transpose(base, (0, 2, 1))[:, :m] = a
    return torch.from_numpy(base).to(device).transpose(1, 2)[:, :m]


def from_dev(t):
    return t.detach().cpu().numpy()


def nrel(X, Xref):
    X = np.asarray(X, dtype=np.complex128)
    Xref = np.asarray(Xref, dtype=np.complex128)
    r = np.linalg.norm(Xref.ravel())
    d = np.linalg.norm((X - Xref).ravel())
    return d / r if r > 0 else d


def max_problem_nrel(X, Xref):
    """Largest per-problem normwise error over a batch."""
    return max(nrel(X[p], Xref[p]) for p in range(X.shape[0]))
