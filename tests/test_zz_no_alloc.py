"""The entry point that allocates nothing, trsm_lln_noalloc, against
trsm_lln on the GPU.

It runs trsm_lln's kernels with the blocked path's workspace taken from the
library's fixed per-device scratch array, so its output must be bitwise that
of trsm_lln (same block size, same kernels), which the oracle bar is then
checked on as well.  Two calls in a row, the second smaller, show that the
contents a call leaves in the shared array do not leak into the next one;
an oversized problem is refused with B untouched.  Called through the C ABI
with ctypes.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import CPLX, TOL, from_dev, nrel, to_dev
from trsm_inputs import CONFIGS, make_config, make_problem

pytestmark = pytest.mark.gpu


def noalloc(T, Ad, Bd, alpha):
    import torch
    code = T._dtype_code(Bd)
    m, n = Bd.shape
    al = T.alpha_buffer(code, alpha)
    return T.lib.trsm_lln_noalloc(code, m, n, ctypes.addressof(al), Ad.data_ptr(), T._ld(Ad, m, m),
                                  Bd.data_ptr(), T._ld(Bd, m, n),
                                  torch.cuda.current_stream().cuda_stream)


def reference(T, Ad, B, alpha):
    import torch
    Bd = to_dev(B)
    T.trsm_lln(Ad, Bd, alpha)
    torch.cuda.synchronize()
    return from_dev(Bd)


# (first call, second smaller call): blocked path, a ragged last block,
# split-K products (narrow B), and the direct path in second place
PAIRS = [
    ("f64", (2000, 1500), (600, 70)),
    ("c64", (1500, 700), (300, 33)),
    ("f32", (3000, 2000), (1000, 257)),
    ("c32", (1200, 900), (100, 5)),
    ("f64", (4000, 40), (2500, 8)),
    ("c64", (2100, 64), (64, 64)),
]


@pytest.mark.parametrize("dtype,first,second", PAIRS)
def test_noalloc_matches_trsm_lln_two_calls(dtype, first, second):
    import torch
    import triangular_solve_trsm_amd as T
    for k, (m, n) in enumerate((first, second)):
        print(f"noalloc {dtype} call {k} m={m} n={n}", flush=True)
        L, B = make_problem(dtype, m, n, seed=500 + 7 * m + n)
        a = 0.75 - 0.25j if dtype in CPLX else 0.75
        Ad = to_dev(L)
        Bd = to_dev(B)
        assert noalloc(T, Ad, Bd, a) == 0
        torch.cuda.synchronize()
        X = from_dev(Bd)
        Xref = reference(T, Ad, B, a)
        assert nrel(X, Xref) <= TOL[dtype]
        assert np.array_equal(X, Xref), f"{dtype} m={m} n={n}: not bitwise trsm_lln's result"
        assert nrel(X, oracle.solve(L, B, a)) <= TOL[dtype]


def test_noalloc_headline_fp64_8192():
    """fp64 m = n = 8192 needs exactly the 128 MiB of the array (ib 1024:
    64 MiB of inverses, 64 MiB of panel); compared on the GPU with
    trsm_lln, bitwise."""
    import torch
    import triangular_solve_trsm_amd as T
    cfg = CONFIGS["c4_f64_8192"]
    L, B, a = make_config(cfg)
    Ad, B0 = to_dev(L), to_dev(B)
    Bd = B0.clone()
    assert noalloc(T, Ad, Bd, a) == 0
    Bref = B0.clone()
    T.trsm_lln(Ad, Bref, a)
    torch.cuda.synchronize()
    assert torch.equal(Bd, Bref)


def test_noalloc_refuses_oversized_problem_untouched():
    """m = 65, n = 2^21 (fp64): the panel alone needs ib * n * 8 bytes, at
    least 1 GiB at any block size, over the 128 MiB array."""
    import torch
    import triangular_solve_trsm_amd as T
    m, n = 65, 1 << 21
    L, _ = make_problem("f64", m, 1, seed=1)
    Ad = to_dev(L)
    Bd = torch.arange(m * n, dtype=torch.float64, device="cuda").reshape(n, m).T
    B0 = Bd.clone()
    assert noalloc(T, Ad, Bd, 1.0) == 1
    torch.cuda.synchronize()
    assert torch.equal(Bd, B0)
    with pytest.raises(T.TrsmError):
        T.trsm_lln_noalloc(Ad, Bd, 1.0)
