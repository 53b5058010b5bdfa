/*
 * trsm.h -- C ABI of a left-side, lower-triangular, non-transposed,
 * non-unit-diagonal TRSM for AMD Instinct MI355X (gfx950).
 *
 * Operation (HSMA-TRSM, "Hierarchical Shared Memory-Aware Optimization for
 * TRSM on GPU Platforms", section 2.1, and the forward-substitution equation
 * of section 4.2.1): given an m x m lower-triangular L (the lower triangle of
 * A, diagonal included) and an m x n B, overwrite B with the X that solves
 *
 *     L X = alpha B,   x_ij = (alpha b_ij - sum_{k<i} l_ik x_kj) / l_ii.
 *
 * Data layout: column-major; element (i, j) of A is A[i + j*lda] and of B is
 * B[i + j*ldb].  Complex data are interleaved (re, im) pairs: of doubles for
 * TRSM_C64F (layout-compatible with hipDoubleComplex), of floats for
 * TRSM_C32F (hipFloatComplex); no operand is conjugated.
 *
 * Ownership: A and B are device pointers owned by the caller, who keeps them
 * alive until the work enqueued on `stream` has completed.  alpha is a host
 * pointer to one scalar of the data type, read before the call returns.
 * `stream` is a hipStream_t (NULL = the default stream); every call only
 * enqueues work on it and returns without waiting.
 *
 * A is read only in its lower triangle (diagonal included): the strict upper
 * triangle and the rows between m and lda are never referenced, so they may
 * hold anything.  B's rows between m and ldb are left untouched.
 *
 * Errors: every argument is checked before any HIP call; on a bad argument
 * nothing is enqueued and B is untouched.  No exception crosses this ABI and
 * the library never aborts.  There is no singularity check (BLAS
 * convention): a zero on the diagonal yields Inf/NaN in X.
 *
 * Workspace: the blocked path (m > 64) needs device scratch space for the
 * inverted diagonal blocks, one panel of B and, when B is narrow, the
 * partial sums of products split along K (at most 2^21 elements).  The
 * library allocates it per (device, stream), grows it on demand and keeps
 * it until trsm_release_workspace().  Calls on the same stream share it:
 * a call holds the stream's workspace from the moment it takes it until
 * it has enqueued its last kernel, so calls from several host threads on
 * one stream are serialised while they enqueue (growth waits for the
 * stream before freeing the old buffer); calls on different streams each
 * get their own workspace and run concurrently.
 */
#ifndef TRSM_MI355X_H
#define TRSM_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's own hipStream_t. */
typedef struct ihipStream_t *hipStream_t;

typedef enum trsm_status_t {
    TRSM_STATUS_SUCCESS = 0,
    TRSM_STATUS_INVALID_VALUE = 1, /* bad dtype/size/leading dimension/pointer */
    TRSM_STATUS_ALLOC_FAILED = 2,  /* workspace could not be allocated       */
    TRSM_STATUS_HIP_ERROR = 3,     /* a HIP runtime call or launch failed     */
    TRSM_STATUS_NOT_SUPPORTED = 4  /* device is not gfx950, or bad option     */
} trsm_status_t;

typedef enum trsm_dtype_t {
    TRSM_R32F = 0, /* float                                   */
    TRSM_R64F = 1, /* double                                  */
    TRSM_C64F = 2, /* complex double, interleaved (re, im)    */
    TRSM_C32F = 3  /* complex float, interleaved (re, im)     */
} trsm_dtype_t;

/*
 * Solve L X = alpha B in place (B <- X).
 *   dtype  TRSM_R32F, TRSM_R64F, TRSM_C64F or TRSM_C32F.
 *   m, n   rows of B (= order of L) and columns of B; m, n >= 0.
 *   alpha  host pointer to one float / double / double[2] (re, im) /
 *          float[2] (re, im), by dtype.
 *   A      device pointer, m x m, lda >= max(1, m).
 *   B      device pointer, m x n, ldb >= max(1, m); overwritten with X.
 *   Every leading dimension the rules above allow is supported, however
 *   large (a sub-block of a tall array): tiles whose columns span more than
 *   a 32-bit offset reaches are read through 64-bit addresses.
 * Quick returns: m == 0 or n == 0 does nothing; alpha == 0 sets B = 0
 * without reading A.  A, B and alpha may be NULL only when m*n == 0.
 * Regime (section 4.1 of the pages): m <= 64 runs the single-workgroup
 * direct solve (one workgroup per 64 columns); m > 64 runs the blocked
 * path (parallel diagonal-block inversion, then per block row an MFMA
 * GEMM solve and an MFMA GEMM trailing update), with the block size taken
 * from the offline-profiled table (trsm_lln_select_ib).
 */
trsm_status_t trsm_lln(trsm_dtype_t dtype, int64_t m, int64_t n, const void *alpha,
                       const void *A, int64_t lda, void *B, int64_t ldb,
                       hipStream_t stream);

/*
 * Strided batch of independent solves (batched TRSM is named as future work
 * in section 6 of the pages): problem p uses A + p*strideA and B + p*strideB
 * (strides in elements of dtype; complex elements for the complex types) and the
 * common alpha.  strideA >= lda*m and strideB >= ldb*n are not required,
 * but problems must not overlap in B.  batch == 0 is a quick return,
 * batch < 0 is INVALID_VALUE.  m <= 64 launches one grid over all problems;
 * larger m runs the blocked path problem by problem.
 */
trsm_status_t trsm_lln_strided_batched(trsm_dtype_t dtype, int64_t m, int64_t n,
                                       const void *alpha, const void *A, int64_t lda,
                                       int64_t strideA, void *B, int64_t ldb,
                                       int64_t strideB, int64_t batch,
                                       hipStream_t stream);

/*
 * trsm_lln with a forced diagonal block size (section 4.3.2 of the pages:
 * the offline sweep times each candidate).  ib == 0 uses the table; any
 * other value must be 64, 128, 256, 512 or 1024, else INVALID_VALUE.  For m <= 64
 * ib is ignored (direct solve), unless force_blocked != 0, which runs the
 * blocked path at any m > 0.
 */
trsm_status_t trsm_lln_ex(trsm_dtype_t dtype, int64_t m, int64_t n, const void *alpha,
                          const void *A, int64_t lda, void *B, int64_t ldb, int ib,
                          int force_blocked, hipStream_t stream);

/* ---- the general TRSM: every side, triangle, transposition, diagonal ---- */

typedef enum trsm_side_t { TRSM_LEFT = 0, TRSM_RIGHT = 1 } trsm_side_t;
typedef enum trsm_fill_t { TRSM_LOWER = 0, TRSM_UPPER = 1 } trsm_fill_t;
typedef enum trsm_op_t { TRSM_OP_N = 0, TRSM_OP_T = 1, TRSM_OP_C = 2 } trsm_op_t;
typedef enum trsm_diag_t { TRSM_NON_UNIT = 0, TRSM_UNIT = 1 } trsm_diag_t;

/*
 * BLAS TRSM (the pages' system op(A) X = alpha B of section 2.1, and its
 * right-side form):
 *   side TRSM_LEFT:  op(A) X = alpha B, A is m x m (lda >= max(1, m));
 *   side TRSM_RIGHT: X op(A) = alpha B, A is n x n (lda >= max(1, n));
 *   uplo: the triangle of A that is used (the other is never read);
 *   trans: op(A) = A, A^T or A^H (TRSM_OP_C; for real types the same as T);
 *   diag TRSM_UNIT: unit diagonal, the diagonal of A is never read.
 *   B: m x n, ldb >= max(1, m), overwritten with X.  Other arguments and the
 *   quick returns as for trsm_lln.
 * trsm_solve(LEFT, LOWER, OP_N, NON_UNIT, ...) is trsm_lln.  Every other case is brought to
 * it by index reflection: the triangle of op(A) (or op(A)^T for the right
 * side) is copied, transposed, conjugated or reversed as needed, into a
 * library workspace (order^2 elements) and solved there; when the
 * right-hand sides need reordering too, B is staged there as well (m*n
 * elements more) and copied back.  The staging workspace is cached per
 * (device, stream) beside the solve's and freed by trsm_release_workspace.
 */
trsm_status_t trsm_solve(trsm_side_t side, trsm_fill_t uplo, trsm_op_t trans, trsm_diag_t diag,
                         trsm_dtype_t dtype, int64_t m, int64_t n, const void *alpha,
                         const void *A, int64_t lda, void *B, int64_t ldb, hipStream_t stream);

/*
 * trsm_lln for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that
 * forbid allocation.  Same arguments, results and quick returns as
 * trsm_lln (the same kernels with the same block size, so X is bitwise that
 * of trsm_lln).  The blocked path's workspace (m > 64) comes from a fixed
 * array in the library's device memory, TRSM_NOALLOC_MAX_WORKSPACE_BYTES
 * per device, held from library load until the process ends; the call
 * performs no allocation of any kind.
 * A problem whose workspace exceeds that size returns
 * TRSM_STATUS_INVALID_VALUE before any HIP call, with B untouched.  The
 * workspace is nb*ib*ib elements of inverses plus max(ib*n, the
 * inversion's scratch) elements of panel plus split-K partial sums (at
 * most 2^21 elements), each rounded up to 256 bytes, with ib and nb =
 * ceil(m/ib) from trsm_lln_select_ib; e.g. fp64 m = n = 8192 (ib 1024)
 * needs 128 MiB and fits, complex fp64 8192 x 2048 needs 160 MiB and does
 * not.  m <= 64 and alpha == 0 need no workspace at all.
 * Every call on one device shares that device's array and leaves its
 * contents behind (nothing in it needs to start at zero): calls whose
 * kernels may overlap in time on one device -- on different streams, or
 * from several host threads without ordering -- race on it and give wrong
 * results.  Calls ordered on one stream are safe.
 */
#define TRSM_NOALLOC_MAX_WORKSPACE_BYTES (128ull << 20)
trsm_status_t trsm_lln_noalloc(trsm_dtype_t dtype, int64_t m, int64_t n, const void *alpha,
                               const void *A, int64_t lda, void *B, int64_t ldb,
                               hipStream_t stream);

/*
 * Block size the blocked path uses for (dtype, m, n): nearest-scale match
 * in the table built by offline profiling on MI355X (section 4.3.2), the
 * scale being (m, n) compared in log space (the table holds square
 * problems and narrow ones, n = 64, 256, 1024).
 * Returns 0 for an invalid dtype or negative size.  Pure, thread-safe.
 */
int trsm_lln_select_ib(trsm_dtype_t dtype, int64_t m, int64_t n);

/* Static description of a status code.  Pure, thread-safe. */
const char *trsm_status_string(trsm_status_t status);

/*
 * Free every cached workspace on every device after waiting for the
 * streams that used them.  Thread-safe; later calls re-allocate.
 */
trsm_status_t trsm_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* TRSM_MI355X_H */
