"""GPU checks of the step-level entry points (include/trsm_kernels.h).

* trsm_kernel_gemm (the phase-2 GEMM of the blocked algorithm) against a
  float64 / complex128 numpy product, element by element, within the
  standard rounding bound of a K-term dot product:
      |D - D_ref| <= 2 (K + 2) u (|beta| |C| + |gamma| |A| |Bm|)   (per element)
  on ragged shapes, odd leading dimensions, the split routing to D2, the
  triangular skip, every macro-tile size, K = 0 and gamma = 0.
* trsm_kernel_diag_inv (phase 1) against the oracle solving each diagonal
  block against the columns of the identity, which is the definition of the
  inverse the pages build the kernel on (section 4.3.1, the identity tile
  E_j as right-hand side).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import NP, from_dev, to_dev
from trsm_inputs import make_problem

pytestmark = pytest.mark.gpu

U = {"f32": 2.0 ** -24, "f64": 2.0 ** -53, "c64": 2.0 ** -53, "c32": 2.0 ** -24}
CPLX = ("c64", "c32")


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import triangular_solve_trsm_amd as T
    return T


def rand(dtype, rows, cols, rng, ld=None):
    if dtype in CPLX:
        a = rng.uniform(-1, 1, (rows, cols)) + 1j * rng.uniform(-1, 1, (rows, cols))
    else:
        a = rng.uniform(-1, 1, (rows, cols))
    a = a.astype(NP[dtype])
    ld = rows if ld is None else ld
    base = np.full((cols, max(ld, 1)), np.nan, dtype=NP[dtype])
    base.T[:rows] = a
    return base.T[:rows]


def gemm_case(T, dtype, M, N, K, beta, gamma, *, seed=0, ldpad=0, split=0, a_lower=False,
              ldpad_a=None, ldpad_b=None):
    import torch
    rng = np.random.default_rng(seed)
    pa = ldpad if ldpad_a is None else ldpad_a
    pb = ldpad if ldpad_b is None else ldpad_b
    A = rand(dtype, M, K, rng, M + pa)
    if a_lower:
        A = np.asfortranarray(np.tril(A))
        A = rand_like_ld(A, M + pa)
    Bm = rand(dtype, K, N, rng, K + pb)
    C = rand(dtype, M, N, rng, M + ldpad)
    Ad, Bd, Cd = to_dev(A), to_dev(Bm), to_dev(C)
    Dd = to_dev(np.full((M, N), np.nan, dtype=NP[dtype], order="F"), ld=M + ldpad)
    D2d = to_dev(np.full((max(split, 1), N), np.nan, dtype=NP[dtype], order="F")) if split else None
    T.trsm_kernel_gemm(Ad, Bd, Dd, beta=beta, gamma=gamma, C=Cd if beta != 0 else None,
                       D2=D2d, split=split, a_lower=a_lower)
    torch.cuda.synchronize()
    D = from_dev(Dd)
    if split:
        D = D.copy()
        D[:split] = from_dev(D2d)[:split]
    wide = np.complex128 if dtype in CPLX else np.float64
    A64, B64, C64 = A.astype(wide), Bm.astype(wide), C.astype(wide)
    ref = gamma * (A64 @ B64) + (beta * C64 if beta != 0 else 0)
    scale = abs(gamma) * (np.abs(A64) @ np.abs(B64)) + (abs(beta) * np.abs(C64) if beta != 0 else 0)
    bound = 2 * (K + 2) * U[dtype] * scale + 1e-300
    err = np.abs(D.astype(wide) - ref)
    assert np.all(np.isfinite(D)), f"non-finite output {dtype} {M}x{N}x{K}"
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert worst <= 1.0, f"{dtype} M={M} N={N} K={K}: error {worst:.2f} x the rounding bound"
    return worst


def rand_like_ld(a, ld):
    rows, cols = a.shape
    base = np.full((cols, max(ld, 1)), np.nan, dtype=a.dtype)
    base.T[:rows] = a
    return base.T[:rows]


SHAPES = [(1, 1, 1), (17, 33, 5), (130, 129, 37), (64, 64, 64), (200, 70, 257), (513, 300, 48)]


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_gemm_ragged_shapes(T, dtype):
    for i, (M, N, K) in enumerate(SHAPES):
        for beta, gamma in [(0.0, 1.0), (1.0, -1.0), (0.5, -1.0), (-2.0, 0.75)]:
            if dtype in CPLX:
                beta, gamma = complex(beta, 0.25 if beta else 0.0), complex(gamma, -0.5)
            gemm_case(T, dtype, M, N, K, beta, gamma, seed=i)


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_gemm_large_tile_path(T, dtype):
    """Enough tiles (>= 1024) to take the large macro tile (fp64 128 x 64,
    complex 64 x 128), with a ragged K tile and odd leading dimensions
    (unaligned 16-byte loads)."""
    M = 1450 if dtype in CPLX else 2900
    gemm_case(T, dtype, M, 2900, 45, 1.0, -1.0, seed=3)
    gemm_case(T, dtype, M, 2900, 40, 0.0, 1.0, seed=4, ldpad=3)


def test_gemm_fp64_128x128_tile(T):
    """fp64 products whose 128 x 128 tiles fill rounds of 512 (here exactly
    512) with 16-byte aligned operands take the 128 x 128 tile: ragged M
    (2000) and N (4000), even K with a ragged last K tile (46, 302), beta 0
    and 1."""
    gemm_case(T, "f64", 2000, 4000, 46, 1.0, -1.0, seed=5)
    gemm_case(T, "f64", 2000, 4000, 302, 0.0, 0.5, seed=6)


LF_CASES = [
    # (M, N, K, ldpad, split, beta, gamma): 16 x 32 = 512 tiles of 128 x 128,
    # 16-byte aligned operands (even leading dimensions)
    (2000, 4000, 0, 0, 0, 1.5, -1.0),      # K = 0: D = beta C
    (2000, 4000, 1, 1, 0, 1.0, -1.0),      # a single k
    (2000, 4000, 7, 1, 0, 0.0, 0.5),
    (2000, 4000, 8, 0, 0, 1.0, -1.0),      # one full chunk
    (2000, 4000, 9, 1, 0, 1.0, -1.0),
    (2000, 4000, 23, 1, 0, -0.5, 2.0),
    (2000, 4000, 46, 2, 0, 1.0, -1.0),     # NaN in the rows of Bm past K
    (1999, 4000, 63, 1, 0, 1.0, -1.0),     # odd M: a row pair split at the edge
    (2000, 4000, 64, 0, 100, 1.0, -1.0),   # rows below 100 routed to D2
    (2000, 4000, 1001, 1, 37, 0.5, -1.0),  # odd split
    (2000, 3999, 128, 0, 0, 1.0, -1.0),    # ragged N
]


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("case", LF_CASES)
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_gemm_lds_free_edges(T, dtype, case, lf, monkeypatch):
    """fp64 and fp32 products that fill the chip with 128 x 128 tiles run the
    LDS-free kernels (each wave streams its own operands into a register
    ring; TRSM_GEMM_LF=0 runs the LDS-staged tiles instead, so both are
    checked): every K modulo the chunk (8 k for fp64, 16 for fp32), K = 0,
    NaN stored right past K in Bm (the ragged chunk must read zeros there),
    odd M, ragged N, the D2 split (even and odd) and several beta / gamma."""
    monkeypatch.setenv("TRSM_GEMM_LF", lf)
    M, N, K, ldpad, split, beta, gamma = case
    # leading dimensions of A and Bm padded to 16-byte aligned columns
    per = 2 if dtype == "f64" else 4
    pa = ldpad + (-(M + ldpad)) % per
    pb = ldpad + (-(K + ldpad)) % per
    gemm_case(T, dtype, M, N, K, beta, gamma, seed=K + M, ldpad=ldpad, ldpad_a=pa, ldpad_b=pb,
              split=split)


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("case", LF_CASES)
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_gemm_lds_free_256_tiles(T, dtype, case, lf, monkeypatch):
    """fp32 and fp64 products with 256 to 511 tiles of 128 x 128 (here 8 x 32
    = 256) take the LDS-free kernels on half-width workgroups, two per CU,
    with a ring of three chunks (fp32: the ring of five above 512): the
    same edge cases as above on half the rows."""
    monkeypatch.setenv("TRSM_GEMM_LF", lf)
    M, N, K, ldpad, split, beta, gamma = case
    M = M // 2
    per = 2 if dtype == "f64" else 4
    pa = ldpad + (-(M + ldpad)) % per
    pb = ldpad + (-(K + ldpad)) % per
    gemm_case(T, dtype, M, N, K, beta, gamma, seed=K + M + 1, ldpad=ldpad, ldpad_a=pa, ldpad_b=pb,
              split=min(split, M))


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("M,N", [(1000, 4000), (960, 4096), (1023, 4000), (1024, 3970), (1024, 2048),
                                 (999, 1100)])
def test_gemm_lds_free_triangular_f32_256(T, M, N, lf, monkeypatch):
    """Triangular fp32 products with 256 folded workgroups (8 pairs of row
    tiles x 32 column blocks) and with 64 to 255 (N = 2048, 1100) on the ring
    of three: ragged last row tile, an odd tile count, odd M, ragged N."""
    monkeypatch.setenv("TRSM_GEMM_LF", lf)
    pa = (-M) % 4
    gemm_case(T, "f32", M, N, M, 0.0, -0.75, seed=M + N + 1, a_lower=True, ldpad_a=pa, ldpad_b=pa)


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("M,N,beta,split,pad", [(1024, 4096, 0.0, 0, 0), (1000, 4000, 0.0, 0, 1),
                                                (960, 4096, 1.5, 0, 0), (1023, 3999, -0.5, 130, 2),
                                                (1024, 2048, 0.0, 0, 0), (1000, 2047, 1.0, 37, 1)])
def test_gemm_lds_free_triangular_f64_256(T, M, N, beta, split, pad, lf, monkeypatch):
    """fp64 triangular products with 256 to 511 folded workgroups of 128
    columns on the LDS-free ring of three, and with fewer (N = 2048) on 64
    columns per workgroup (TRSM_GEMM_LF=0: the LDS tile): ragged last row
    tile, odd tile count, odd M and N, a C term, rows routed to D2 below a
    split inside a row pair."""
    monkeypatch.setenv("TRSM_GEMM_LF", lf)
    print(f"case f64 tri M={M} N={N} beta={beta} split={split} lf={lf}", flush=True)
    gemm_case(T, "f64", M, N, M, beta, -0.75, seed=M + N + split, a_lower=True, split=split,
              ldpad=pad, ldpad_a=pad, ldpad_b=pad)


@pytest.mark.parametrize("form", ["1", "0"])
@pytest.mark.parametrize("M,N,beta,split,pad", [(1024, 2048, 0.0, 0, 0), (1000, 2000, 0.0, 0, 1),
                                                (999, 2048, 1.0 - 0.5j, 0, 0), (1024, 2047, 0.5, 130, 2),
                                                (1024, 1024, 0.0, 0, 0), (999, 1023, 0.5j, 65, 1)])
def test_gemm_lds_free_triangular_complex(T, M, N, beta, split, pad, form, monkeypatch):
    """Complex fp64 triangular products on the LDS-free kernel through the
    real view, 64 x 32 per wave and (N = 1024) 64 x 16 per wave
    (TRSM_LF_CPLX_TRI=0: the LDS tile): a ragged last row tile,
    odd M (complex rows stay whole: a real row pair never straddles two
    tiles), ragged N, a C term, rows routed to D2."""
    monkeypatch.setenv("TRSM_LF_CPLX_TRI", form)
    print(f"case c64 tri M={M} N={N} beta={beta} split={split} form={form}", flush=True)
    gemm_case(T, "c64", M, N, M, beta, -0.75 + 0.25j, seed=M + N + split, a_lower=True, split=split,
              ldpad=pad, ldpad_a=pad, ldpad_b=pad)


LF_CPLX_CASES = [
    # (M, N, K, ldpad, split, beta, gamma) in complex elements: the real view
    # 2M x N gives 16 x 32 = 512 tiles of 128 x 128
    (1000, 4000, 0, 0, 0, 1.5 - 0.5j, -1.0),        # K = 0: D = beta C
    (1000, 4000, 1, 1, 0, 1.0, -1.0 + 0.5j),        # a single k
    (1000, 4000, 3, 1, 0, 0.0, 0.5j),
    (1000, 4000, 4, 0, 0, 1.0, -1.0),               # one full chunk (8 real k)
    (1000, 4000, 5, 1, 0, 0.25j, -1.0),
    (1000, 4000, 23, 2, 0, -0.5 + 1j, 2.0 - 1j),    # NaN in the rows of Bm past K
    (999, 4000, 31, 1, 0, 1.0, -1.0),               # odd M
    (1000, 4000, 64, 0, 100, 1.0, -1.0),            # rows below 100 routed to D2
    (1000, 4000, 501, 1, 37, 0.5 + 0.25j, -1.0),    # odd split
    (1000, 3999, 128, 0, 0, 1.0, -1.0 - 1j),        # ragged N
]


@pytest.mark.parametrize("K,beta,split,pad", [(0, 1.5, 0, 0), (1, 1.0, 0, 1), (15, 0.0, 0, 2), (16, 1.0, 0, 0),
                                          (17, -0.5, 100, 1), (100, 1.0, 37, 3), (2048, 1.0, 0, 0),
                                          (2063, 0.5, 64, 1), (3000, 0.0, 0, 2)])
def test_gemm_lds_free_f32_k_split(T, K, beta, split, pad, monkeypatch):
    """fp32 products with 256 to 511 tiles of 128 x 128 and a long K run on
    eight-wave workgroups whose two halves of K meet through LDS (forced
    here from K = 1 with TRSM_LF32_KS=1): an empty first half (K < 32), K a
    multiple of the chunk, ragged K (the second half takes the ragged
    chunk), a C term, the D2 split, NaN past K in Bm."""
    monkeypatch.setenv("TRSM_LF32_KS", "1")
    M, N = 1000, 4000
    pa = pad + (-(M + pad)) % 4
    pb = pad + (-(K + pad)) % 4
    print(f"case f32 k-split M={M} N={N} K={K} split={split}", flush=True)
    gemm_case(T, "f32", M, N, K, beta, -1.0, seed=K + 7, ldpad=pad, ldpad_a=pa, ldpad_b=pb, split=split)


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("case", LF_CASES)
@pytest.mark.parametrize("dtype", ["f32", "f64", "c64"])
def test_gemm_lds_free_64_tiles(T, dtype, case, lf, monkeypatch):
    """fp32, fp64 and complex fp64 products with 64 to 255 tiles of 128 x 128
    (here a quarter of the rows: 4 x 32 = 128; the real view of complex the
    same) on 128 x 32 LDS-free workgroups: the edge cases above."""
    monkeypatch.setenv("TRSM_GEMM_LF", lf)
    M, N, K, ldpad, split, beta, gamma = case
    M = M // 8 if dtype == "c64" else M // 4
    per = {"f32": 4, "f64": 2, "c64": 1}[dtype]
    pa = ldpad + (-(M + ldpad)) % per
    pb = ldpad + (-(K + ldpad)) % per
    if dtype == "c64":
        beta, gamma = beta * (1 - 0.5j), gamma * (0.5 + 1j)
    gemm_case(T, dtype, M, N, K, beta, gamma, seed=K + M + 3, ldpad=ldpad, ldpad_a=pa, ldpad_b=pb,
              split=min(split, M))


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("div", [1, 2, 8])
@pytest.mark.parametrize("case", LF_CPLX_CASES)
def test_gemm_lds_free_complex_f32(T, case, div, lf, monkeypatch):
    """Complex fp32 products on the LDS-free fp32 kernel through the real
    view (one 16-byte A load feeds two MFMA steps as (re, im) and (-im, re);
    TRSM_LF_C32=0: the LDS tiles), at 512, 256 and 64 tiles of 128 x 128
    (the cases below on all, half and an eighth of the rows): every K
    modulo the chunk (8 complex k), K = 0, NaN past K in Bm, odd M, ragged
    N, the D2 split, complex beta and gamma."""
    monkeypatch.setenv("TRSM_LF_C32", lf)
    M, N, K, ldpad, split, beta, gamma = case
    M = M // div
    print(f"case c32 M={M} N={N} K={K} split={split} lf={lf}", flush=True)
    gemm_case(T, "c32", M, N, K, beta, gamma, seed=K + M + 5, ldpad=ldpad, split=min(split, M))


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("M,N,beta,split,pad", [(1000, 4000, 0.0, 0, 0), (1024, 2048, 0.5j, 0, 1),
                                                (999, 1024, 0.0, 65, 0), (500, 4096, 1.0, 0, 2)])
def test_gemm_lds_free_triangular_c32(T, M, N, beta, split, pad, lf, monkeypatch):
    """Complex fp32 triangular products on the LDS-free fp32 forms through
    the real view (folded pairs of 64 real rows; 512, 256 and 128 folded
    workgroups of 128 columns), against the LDS tiles (TRSM_LF_C32=0)."""
    monkeypatch.setenv("TRSM_LF_C32", lf)
    print(f"case c32 tri M={M} N={N} beta={beta} split={split} lf={lf}", flush=True)
    gemm_case(T, "c32", M, N, M, beta, -0.75 + 0.25j, seed=M + N + split, a_lower=True, split=split,
              ldpad=pad, ldpad_a=pad, ldpad_b=pad)


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("case", LF_CPLX_CASES)
def test_gemm_lds_free_complex_256_tiles(T, case, lf, monkeypatch):
    """Complex fp64 products whose real view gives 256 to 511 tiles of
    128 x 128 (here 8 x 32) on half-width LDS-free workgroups, two per CU:
    the cases below on half the complex rows."""
    monkeypatch.setenv("TRSM_GEMM_LF", lf)
    M, N, K, ldpad, split, beta, gamma = case
    M = M // 2
    gemm_case(T, "c64", M, N, K, beta, gamma, seed=K + M + 2, ldpad=ldpad, split=min(split, M))


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("case", LF_CPLX_CASES)
def test_gemm_lds_free_complex(T, case, lf, monkeypatch):
    """Complex fp64 products that fill the chip run the LDS-free fp64 kernel
    on their real view (each complex element of A the 2 x 2 block [[re, -im],
    [im, re]], Bm, C and D read as interleaved real; TRSM_GEMM_LF=0: the LDS
    tiles): every K modulo the chunk (4 complex k), K = 0, NaN right past K
    in Bm, odd M, ragged N, the D2 split, complex beta and gamma (C and the
    result scaled as complex numbers)."""
    monkeypatch.setenv("TRSM_GEMM_LF", lf)
    M, N, K, ldpad, split, beta, gamma = case
    gemm_case(T, "c64", M, N, K, beta, gamma, seed=K + M, ldpad=ldpad, split=split)


@pytest.mark.parametrize("lf", ["1", "0"])
@pytest.mark.parametrize("M,N", [(1000, 8100), (960, 8192), (1023, 8192), (1024, 8190)])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_gemm_lds_free_triangular(T, dtype, M, N, lf, monkeypatch):
    """Triangular fp64 and fp32 products with at least 512 workgroups run the
    LDS-free form (TRSM_GEMM_LF=0: the LDS tile): each wave takes the 64-row tiles i
    and T-1-i of a 32-column block, each over K up to its own diagonal.
    Ragged last row tile (1000 = 15 x 64 + 40), an odd count of row tiles
    (960: the middle tile runs alone), odd M (a row pair split at the edge),
    ragged N."""
    monkeypatch.setenv("TRSM_GEMM_LF", lf)
    pa = (-M) % (2 if dtype == "f64" else 4)  # 16-byte aligned columns
    gemm_case(T, dtype, M, N, M, 0.0, -0.75, seed=M + N, a_lower=True, ldpad_a=pa, ldpad_b=pa)


@pytest.mark.parametrize("dtype", ["f64", "c64"])
def test_gemm_triangular_wide_tiles(T, dtype):
    """Triangular products with 512 folded workgroups on the wider tile
    (fp64 64 x 128, complex 64 x 64): ragged M (1000 rows, the last row tile
    short) and ragged N."""
    N = 8100 if dtype == "f64" else 2000
    gemm_case(T, dtype, 1000, N, 1000, 0.0, 0.5 if dtype == "f64" else 0.5 - 0.25j, seed=12, a_lower=True)


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_gemm_split_routing(T, dtype):
    for split in (16, 37, 100):
        gemm_case(T, dtype, 300, 90, 64, 1.0, -1.0, seed=split, split=split)


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
def test_gemm_triangular(T, dtype):
    for M in (64, 100, 256, 300):
        gemm_case(T, dtype, M, 150, M, 0.0, 0.5, seed=M, a_lower=True)


@pytest.mark.parametrize("dtype", ["f64", "c64", "c32"])
def test_gemm_k_zero_and_gamma_zero(T, dtype):
    gemm_case(T, dtype, 50, 40, 0, 1.5, -1.0, seed=1)
    gemm_case(T, dtype, 50, 40, 30, 1.5, 0.0, seed=2)


@pytest.mark.parametrize("dtype", ["f32", "f64", "c64", "c32"])
@pytest.mark.parametrize("ib", [64, 128, 256, 512, 1024])
def test_diag_inv_vs_oracle_identity_solve(T, dtype, ib):
    diag_inv_case(T, dtype, ib, ib * 2 + 37)  # two full blocks and a ragged one


@pytest.mark.parametrize("dtype,lf", [("f32", None), ("f64", "1"), ("f64", "0"), ("c64", "1"), ("c64", "0")])
@pytest.mark.parametrize("ib,m", [(256, 3 * 256 + 200), (512, 2 * 512 + 300), (1024, 3 * 1024), (1024, 2048 + 777)])
def test_diag_inv_doubling_pairs(T, dtype, ib, m, lf, monkeypatch):
    """Batched doubling products over several parent blocks: full pairs in
    every block, a last block with no ragged rows, and ragged last blocks
    whose last pair is cut short at different levels.  fp64 and complex
    fp64 run every level's products on the LDS-free kernel
    (TRSM_INV_LF_MIN=1; complex through the real view) and on the LDS tile
    (TRSM_INV_LF=0)."""
    if lf == "1":
        monkeypatch.setenv("TRSM_INV_LF_MIN", "1")
    elif lf == "0":
        monkeypatch.setenv("TRSM_INV_LF", "0")
    print(f"case {dtype} ib={ib} m={m} lf={lf}", flush=True)
    diag_inv_case(T, dtype, ib, m)


def diag_inv_case(T, dtype, ib, m):
    import torch
    L, _ = make_problem(dtype, m, 1, seed=ib)
    nb = (m + ib - 1) // ib
    W = torch.full((nb * ib * ib,), float("nan"), dtype={"f32": torch.float32, "f64": torch.float64,
                                                         "c64": torch.complex128, "c32": torch.complex64}[dtype],
                    device="cuda")
    T.trsm_kernel_diag_inv(to_dev(L), W, ib)
    torch.cuda.synchronize()
    Wh = from_dev(W)
    tol = 1e-5 if dtype in ("f32", "c32") else 1e-13
    for t in range(nb):
        r0 = t * ib
        bs = min(ib, m - r0)
        D = np.asfortranarray(L[r0:r0 + bs, r0:r0 + bs])
        ref = oracle.solve(D, np.asfortranarray(np.eye(bs, dtype=D.dtype)), 1.0)
        Wt = Wh[t * ib * ib:(t + 1) * ib * ib].reshape(ib, ib).T[:bs, :bs]
        assert np.all(np.triu(Wt, 1) == 0), "upper triangle of the inverse must be explicit zeros"
        e = np.linalg.norm(Wt - ref) / np.linalg.norm(ref)
        assert e <= tol, (dtype, ib, t, e)


def test_profile_records_by_kind(T):
    """The launch profiler records every launch of a blocked solve with
    HIP events (kind, sizes, duration), and only the selected kinds after
    trsm_profile_select."""
    import torch
    L, B = make_problem("f64", 700, 90, seed=4)
    Ad, Bd = to_dev(L), to_dev(B)
    T.trsm_profile_select(None)
    T.trsm_profile_start()
    T.trsm_lln_ex(Ad, Bd, 1.0, ib=128)
    torch.cuda.synchronize()
    T.trsm_profile_stop()
    kinds = [r["kind"] for r in T.profile_records()]
    assert kinds[0] == "diag_inv" and "copy" in kinds and "update_gemm" in kinds
    assert kinds.count("solve_gemm") == 6  # ceil(700 / 128) block rows
    assert all(r["ms"] > 0 for r in T.profile_records())
    T.trsm_profile_select(["update_gemm"])
    T.trsm_profile_start()
    T.trsm_lln_ex(Ad, Bd, 1.0, ib=128)
    torch.cuda.synchronize()
    T.trsm_profile_stop()
    T.trsm_profile_select(None)
    recs = T.profile_records()
    assert recs and all(r["kind"] == "update_gemm" for r in recs)
