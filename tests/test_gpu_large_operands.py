"""GPU parity at the largest operand sizes the offsets have to carry.

The kernels address operands through 32-bit buffer offsets taken from a
per-tile (or per-problem) base, and index the rest in 64 bits; launch grids
are capped at 65535 blocks in y.  These cases put a right-hand side past
2 GiB and past 4 GiB, and a reflected operand past 65535 column tiles:

* the blocked path, fp64 m = 100, n = 5.5 M (B is 4.4 GB);
* the direct path (m <= 64), fp64 m = 64, n = 4.3 M (B is 2.2 GB: one
  problem wider than a 32-bit buffer range takes the guarded loads);
* trsm_solve on the right side, m = 2.2 M rows of B against a 64 x 64
  upper A (the right-hand sides, staged transposed, are 2.2 M columns).

Right-hand sides are independent (column j of X depends only on A and
column j of B for a left solve; row i for a right solve), so each case is
compared element by element with the oracle on sampled columns (rows) at the
start, the end and on both sides of the 2^31 and 2^32 byte offsets, and the
whole output is checked by the residual ||op(A) X - alpha B|| computed by
torch on the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import TOL, nrel
from trsm_inputs import make_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import triangular_solve_trsm_amd as T
    return T


def draw_colmajor(rng, m, n):
    """uniform[-1, 1] (m, n) array in column-major order, drawn in chunks of
    columns to bound the temporaries."""
    out = np.empty((n, m))
    step = 1 << 19
    for s in range(0, n, step):
        out[s:s + step] = rng.uniform(-1, 1, (min(step, n - s), m))
    return out.T


def sample_indices(count, bytes_per_index):
    """Indices at the ends and on both sides of the 2^31 and 2^32 byte offsets."""
    idx = {0, 1, count // 2, count - 2, count - 1}
    for edge in (1 << 31, 1 << 32):
        j = edge // bytes_per_index
        idx.update(k for k in (j - 1, j, j + 1) if 0 <= k < count)
    return np.array(sorted(idx))


def residual(A_dev_op, X_dev, B_dev, alpha, left=True):
    import torch
    R = (A_dev_op @ X_dev if left else X_dev @ A_dev_op) - alpha * B_dev
    return float(torch.linalg.norm(R) / (torch.linalg.norm(A_dev_op) * torch.linalg.norm(X_dev)
                                         + abs(alpha) * torch.linalg.norm(B_dev)))


def run_left(T, m, n, seed, alpha):
    import torch
    L, _ = make_problem("f64", m, 1, seed=seed)
    B = draw_colmajor(np.random.default_rng(seed + 1), m, n)
    Ad = torch.from_numpy(np.ascontiguousarray(L.T)).cuda().T
    B0 = torch.from_numpy(B.T).cuda().T          # column-major, ld = m
    Bd = B0.clone(memory_format=torch.preserve_format)
    assert Bd.stride() == (1, m)
    T.trsm_lln(Ad, Bd, alpha)
    torch.cuda.synchronize()
    cols = sample_indices(n, m * 8)
    X = Bd[:, torch.as_tensor(cols, device="cuda")].cpu().numpy()
    ref = oracle.solve(L, np.asfortranarray(B[:, cols]), alpha)
    e = nrel(X, ref)
    assert e <= TOL["f64"], f"m={m} n={n}: sampled columns, error {e:.3e}"
    r = residual(torch.tril(Ad.contiguous()), Bd, B0, alpha)
    assert r <= 10 * m * 2.0 ** -53, f"m={m} n={n}: residual {r:.3e}"
    return e, r


def test_blocked_path_b_past_4gib(T):
    e, r = run_left(T, 100, 5_500_000, seed=41, alpha=0.5)
    print(f"blocked m=100 n=5.5M: sampled error {e:.2e}, residual {r:.2e}")


def test_direct_path_one_problem_past_2gib(T):
    e, r = run_left(T, 64, 4_300_000, seed=43, alpha=-1.5)
    print(f"direct m=64 n=4.3M: sampled error {e:.2e}, residual {r:.2e}")


def test_right_side_variant_past_65535_column_tiles(T):
    import torch
    m, k, alpha = 2_200_000, 64, 0.75
    rng = np.random.default_rng(47)
    A = rng.uniform(-1, 1, (k, k)) / k + np.diag(rng.uniform(1, 2, k))
    A = np.asfortranarray(np.triu(A))
    B = draw_colmajor(rng, m, k)
    Ad = torch.from_numpy(np.ascontiguousarray(A.T)).cuda().T
    B0 = torch.from_numpy(B.T).cuda().T
    Bd = B0.clone(memory_format=torch.preserve_format)
    T.trsm_solve(Ad, Bd, alpha, side="R", uplo="U", trans="N", diag="N")
    torch.cuda.synchronize()
    rows = sample_indices(m, 8)
    X = Bd[torch.as_tensor(rows, device="cuda"), :].cpu().numpy()
    ref = oracle.trsm("R", "U", "N", "N", A, np.asfortranarray(B[rows, :]), alpha)
    e = nrel(X, ref)
    assert e <= TOL["f64"], f"right side m={m}: sampled rows, error {e:.3e}"
    r = residual(Ad, Bd, B0, alpha, left=False)
    assert r <= 10 * k * 2.0 ** -53, f"right side m={m}: residual {r:.3e}"
    print(f"right side m=2.2M: sampled error {e:.2e}, residual {r:.2e}")
