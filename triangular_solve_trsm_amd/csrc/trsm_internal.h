// Internal interfaces between the host dispatcher (api.cpp) and the gfx950
// kernels (small_lln.hip, diag_inv.hip, gemm_mfma.hip, aux_kernels.hip).
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trsm {

// Element types.  `cplx` is an interleaved (re, im) pair of doubles,
// layout-compatible with hipDoubleComplex.
struct alignas(16) cplx {
    double re, im;
};
// Complex fp32: an interleaved (re, im) pair of floats, layout-compatible
// with hipFloatComplex.
struct alignas(8) cplx32 {
    float re, im;
};

enum DType : int { R32F = 0, R64F = 1, C64F = 2, C32F = 3 };

inline size_t dtype_size(int dt) {
    return dt == R32F ? 4 : (dt == R64F || dt == C32F) ? 8 : 16;
}

// Scalars travel between host and device code as a pair of doubles
// (fp32 values are widened; only `re` is used for real types).
struct Scalar {
    double re, im;
};

// ---- kernel (a): direct solve, m <= 64 -----------------------------------
// One workgroup per (problem, group of 64 right-hand-side columns): fp64 and
// complex fp64 on the matrix cores (small_mfma_launch), fp32 with one
// 16-row panel per wave on the vector units.
hipError_t small_lln_launch(int dtype, int m, int64_t n, Scalar alpha, const void *A,
                            int64_t lda, int64_t strideA, void *B, int64_t ldb,
                            int64_t strideB, int64_t batch, hipStream_t stream);
hipError_t small_mfma_launch(int dtype, int m, int64_t n, Scalar alpha, const void *A,
                             int64_t lda, int64_t strideA, void *B, int64_t ldb,
                             int64_t strideB, int64_t batch, hipStream_t stream);

// ---- kernel (b1): inversion of every ib x ib diagonal block ---------------
// W receives ceil(m/ib) blocks, block t at W + t*ib*ib (column-major, ld ib),
// each lower triangular with explicit zeros above the diagonal.  tmp holds
// diag_inv_tmp_elems(ib, m) elements of scratch (may be null when that is 0);
// it must not overlap W or A.
int64_t diag_inv_tmp_elems(int ib, int64_t m);
hipError_t diag_inv_launch(int dtype, int ib, int64_t m, const void *A, int64_t lda,
                           void *W, void *tmp, hipStream_t stream);

// ---- kernels (b2, b3): MFMA GEMM -----------------------------------------
//   D = beta * C + gamma * (A * Bm)
// A: M x K (lda), Bm: K x N (ldb), C/D: M x N, all column-major.
// Output rows [0, split) go to D2 (ldd2) instead of D (ldd); any 0 <= split <= M
// (a ragged last block row routes fewer than ib rows).
// C may alias D (in place).  beta == 0 means C is not read (may be null).
// a_lower != 0: A is lower triangular (explicit zeros above the diagonal);
// K-tiles to the right of a row tile's diagonal are skipped (requires M == K).
// b_lower != 0: Bm is lower triangular (explicit zeros above the diagonal);
// the K-tiles above a column tile's diagonal are skipped.  Not with a_lower.
// batch > 1: `batch` independent problems of the same shape; problem
// z = zo * binner + zi (0 <= zi < binner) finds its operands at element
// offsets zo * s?o + zi * s?i from the pointers (split must be 0).  With
// a_lower, problem z's A is the column slice that starts zo * sKo columns
// into the triangle: its element (i, k) is zero (explicitly stored) when
// k + zo * sKo > i, and the K-tiles wholly in that part are skipped.  A
// value-initialised descriptor (batch 0) is a single problem.
struct GemmDesc {
    int64_t M, N, K;
    const void *A;
    int64_t lda;
    const void *Bm;
    int64_t ldb;
    const void *C;
    int64_t ldc;
    void *D;
    int64_t ldd;
    void *D2;
    int64_t ldd2;
    int64_t split;
    Scalar beta, gamma;
    int a_lower;
    int b_lower;
    int64_t batch, binner;
    int64_t sAo, sAi, sBo, sBi, sCo, sCi, sDo, sDi;
    int64_t sKo;
};
hipError_t gemm_launch(int dtype, const GemmDesc &g, hipStream_t stream);

// Split-K form of a single (batch <= 1) product, for products with few
// output tiles and a long K, whose few workgroups would each walk the whole
// K range: the K range is cut into `parts` equal chunks, computed by one
// batched launch into `partial` (parts column-major M x N blocks, ld M),
// then D = beta * C + gamma * sum_s partial_s (s ascending, so the result
// does not depend on timing) by a reduction kernel that keeps gemm_launch's
// D/D2 row split.  With a_lower each chunk still skips the K tiles right of
// the diagonal (sKo = chunk length), so a triangular product keeps its
// halved arithmetic.  parts == 1 is plain gemm_launch.
// gemm_splitk_parts picks parts: a power of two with chunks of at least
// kSplitKMinChunk (a multiple of it) and at most target_workgroups tiles of
// 64 x 32 real rows x columns over all chunks; 1 when no split fits or
// N > 65535.
// parts * M * N never exceeds kSplitKMaxElems.
constexpr int64_t kSplitKMinChunk = 128;
constexpr int64_t kSplitKMaxElems = int64_t(1) << 21;
int gemm_splitk_parts(int dtype, int64_t M, int64_t N, int64_t K, int64_t target_workgroups);
hipError_t gemm_splitk_launch(int dtype, const GemmDesc &g, int parts, void *partial,
                              hipStream_t stream);

// ---- auxiliary kernels ----------------------------------------------------
// B[p] <- 0 for an m x n column-major matrix per problem.
hipError_t fill_zero_launch(int dtype, int64_t m, int64_t n, void *B, int64_t ldb,
                            int64_t strideB, int64_t batch, hipStream_t stream);
// dst (rows x n, ldd) <- src (rows x n, lds).
hipError_t copy_panel_launch(int dtype, int64_t rows, int64_t n, const void *src,
                             int64_t lds, void *dst, int64_t ldd, hipStream_t stream);
// Index reflection of an R x C dst from src:
//   dst(i, j) = f(src(a, b)),  a = revR ? R-1-i : i,  b = revC ? C-1-j : j,
// src(a, b) at src[a + b*lds], or at src[b + a*lds] when trans; f conjugates
// when conj (complex types).  lower: only i >= j is read and written.
// unit: dst(i, i) = 1 (src's diagonal is not read).
struct Reflect {
    int revR, revC, trans, conj, lower, unit;
};
// ---- fixed scratch of trsm_lln_noalloc (noalloc.hip) ------------------------
// Device address of the current device `dev`'s copy of the library's static
// scratch array (TRSM_NOALLOC_MAX_WORKSPACE_BYTES), taken on the first call
// for that device; *bytes receives its size.
hipError_t noalloc_scratch(int dev, void **out, size_t *bytes);

hipError_t transform_launch(int dtype, int64_t R, int64_t C, const void *src, int64_t lds,
                            void *dst, int64_t ldd, const Reflect &f, hipStream_t stream);

}  // namespace trsm
