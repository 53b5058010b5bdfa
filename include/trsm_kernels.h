/*
 * trsm_kernels.h -- step-level entry points and launch profiling of the
 * MI355X left-lower TRSM library (companion of trsm.h, same conventions:
 * column-major device operands, host scalars, work enqueued on `stream`,
 * every argument checked before any HIP call, status codes of trsm.h).
 *
 * The blocked algorithm of HSMA-TRSM ("Hierarchical Shared Memory-Aware
 * Optimization for TRSM on GPU Platforms", section 4.3) runs as a sequence
 * of kernels; these entry points launch one step on its own so that tests
 * and measurement tools can check and time each step.
 */
#ifndef TRSM_MI355X_KERNELS_H
#define TRSM_MI355X_KERNELS_H

#include "trsm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Phase 1 (section 4.3 "Phase 1", section 4.3.1, Figures 6-7): invert every
 * ib x ib diagonal block of the lower triangle of A (m x m, lda).
 * W: device buffer of ceil(m/ib)*ib*ib elements; block t is written at
 * W + t*ib*ib, column-major with leading dimension ib, lower triangular with
 * explicit zeros above the diagonal; the last block covers m - t*ib rows and
 * columns (entries outside it are not written).
 * The 64 x 64 diagonal blocks are inverted by substitution (section 4.3.1)
 * and combined into ib x ib inverses by recursive doubling on the matrix
 * cores; for ib > 64 the scratch of that step comes from the library's
 * per-(device, stream) workspace (TRSM_STATUS_ALLOC_FAILED if it cannot
 * grow).
 * ib in {64, 128, 256, 512, 1024}; m >= 0.
 */
trsm_status_t trsm_kernel_diag_inv(trsm_dtype_t dtype, int ib, int64_t m, const void *A,
                                   int64_t lda, void *W, hipStream_t stream);

/*
 * Phase 2 GEMM (section 4.3 "Phase 2"):  D = beta*C + gamma*(A*Bm)
 *   A: M x K (lda >= max(1,M)), Bm: K x N (ldb >= max(1,K)),
 *   C: M x N (ldc >= max(1,M)); C is not read when *beta == 0 (may be NULL);
 *   D: M x N (ldd >= max(1,M)), may equal C (in place).
 *   D2: if not NULL, rows [0, split) of the result go to D2 (ldd2 >= split)
 *       instead of D; 0 <= split <= M.
 *   a_lower != 0: A is lower triangular with explicit zeros above the
 *       diagonal and M == K (the diagonal-block solve); K-tiles right of
 *       the diagonal are skipped.
 *   beta, gamma: host scalars of dtype.
 * D must not overlap A or Bm.
 */
trsm_status_t trsm_kernel_gemm(trsm_dtype_t dtype, int64_t M, int64_t N, int64_t K,
                               const void *beta, const void *gamma, const void *A,
                               int64_t lda, const void *Bm, int64_t ldb, const void *C,
                               int64_t ldc, void *D, int64_t ldd, void *D2, int64_t ldd2,
                               int64_t split, int a_lower, hipStream_t stream);

/* ---- launch profiling -------------------------------------------------- */

typedef enum trsm_kernel_kind_t {
    TRSM_KERNEL_SMALL = 0,       /* direct solve, m <= 64 (kernel a)       */
    TRSM_KERNEL_DIAG_INV = 1,    /* phase 1 diagonal-block inversion       */
    TRSM_KERNEL_COPY = 2,        /* first panel copy into the panel buffer */
    TRSM_KERNEL_SOLVE_GEMM = 3,  /* phase 2 diagonal-block solve GEMM      */
    TRSM_KERNEL_UPDATE_GEMM = 4, /* phase 2 trailing update GEMM           */
    TRSM_KERNEL_FILL = 5         /* alpha == 0 zero fill                   */
} trsm_kernel_kind_t;

/* One launch: kind, dtype, sizes (GEMM: M, N, K; small: m, n, -, batch;
 * diag_inv: m, ib, -, blocks; copy/fill: rows, cols) and its duration in
 * milliseconds between HIP events recorded on the launch's stream. */
typedef struct trsm_profile_record_t {
    int32_t kind;
    int32_t dtype;
    int64_t m, n, k, batch;
    float ms;
} trsm_profile_record_t;

/* Clear the record list and start recording every later launch of the
 * library (all threads, all streams).  Recording adds two event records
 * per launch and nothing else. */
trsm_status_t trsm_profile_start(void);
/* Record only the launches whose kind k has bit k set in kind_mask (from
 * the next launch on; the default is every kind).  Fewer records mean fewer
 * event records on the streams, so a timed region perturbed by profiling
 * can be limited to the kernels it reports. */
trsm_status_t trsm_profile_select(uint32_t kind_mask);
/* Stop recording (records are kept until the next start). */
trsm_status_t trsm_profile_stop(void);
/* Number of recorded launches. */
int64_t trsm_profile_count(void);
/* Copy record i (0-based); waits for that launch to finish. */
trsm_status_t trsm_profile_read(int64_t i, trsm_profile_record_t *rec);

#ifdef __cplusplus
}
#endif

#endif /* TRSM_MI355X_KERNELS_H */
