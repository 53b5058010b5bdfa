/*
 * CPU oracle for left-side, lower-triangular, non-transposed, non-unit TRSM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library or
 * its Python binding) may include, link, load or call this file.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * What it computes (HSMA-TRSM, "Hierarchical Shared Memory-Aware Optimization
 * for TRSM on GPU Platforms", section 2.1 and the forward-substitution
 * equation of section 4.2.1): for an m x m lower-triangular L and an m x n B,
 * X solves L X = alpha B, row by row,
 *
 *     x[i][j] = ( alpha * b[i][j] - sum_{k<i} l[i][k] * x[k][j] ) / l[i][i].
 *
 * The loop order used here is the column ("axpy") order: scale column j of B
 * by alpha, then for k = 0..m-1 divide row k by l[k][k] and subtract
 * l[i][k] * x[k][j] from every later row i.  Each element therefore sees
 * exactly the operation sequence of the formula above (start from alpha*b,
 * subtract the products in ascending k, divide last), so the two orders give
 * bitwise-identical results.  That claim is checked by the test suite against
 * a row-wise dot-form loop (oracle_lln_d_rowdot below).
 *
 * Conventions (BLAS, as the section 2.1 system op(A) X = alpha B implies):
 *   - column-major: element (i, j) of A is A[i + j*lda];
 *   - only the lower triangle of A, diagonal included, is read;
 *   - B is overwritten by X;
 *   - alpha == 0 sets X = 0 and does not read A;
 *   - no singularity check: a zero diagonal yields Inf/NaN.
 *
 * Complex data are interleaved (re, im) pairs of doubles (_z) or of floats
 * (_c, complex fp32, computed in float: the operand precision).  The complex
 * arithmetic is written out in real operations:
 *   (a+bi)(c+di) = (ac - bd) + (ad + bc)i,
 *   (a+bi)/(c+0i) = a/c + (b/c)i                          (imag(divisor) == 0),
 *   (a+bi)/(c+di) = ((ac+bd) + (bc-ad)i) / (c^2 + d^2)    (otherwise).
 *
 * Build: plain C, -O2 -ffp-contract=off (no fused multiply-add, no fast-math),
 * OpenMP over independent right-hand-side columns and over batch entries;
 * results do not depend on the thread count.
 */
#include <stdint.h>
#include <stddef.h>

/* ---- fp64 ------------------------------------------------------------ */

static void solve_column_d(int64_t m, double alpha, const double *A,
                           int64_t lda, double *b)
{
    int64_t i, k;
    if (alpha == 0.0) {
        for (i = 0; i < m; ++i) b[i] = 0.0;
        return;
    }
    for (i = 0; i < m; ++i) b[i] = alpha * b[i];
    for (k = 0; k < m; ++k) {
        const double *lk = A + k * lda;
        double xk = b[k] / lk[k];
        b[k] = xk;
        for (i = k + 1; i < m; ++i) b[i] = b[i] - lk[i] * xk;
    }
}

int oracle_lln_d(int64_t m, int64_t n, double alpha, const double *A,
                 int64_t lda, double *B, int64_t ldb)
{
    int64_t j;
    if (m < 0 || n < 0 || lda < (m > 1 ? m : 1) || ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (j = 0; j < n; ++j) solve_column_d(m, alpha, A, lda, B + j * ldb);
    return 0;
}

/* Row-wise dot form of the same formula: x[i][j] is produced in one go from
 * alpha*b[i][j] minus the ascending-k products, then divided by l[i][i].
 * Kept only to check that the column order above changes nothing. */
int oracle_lln_d_rowdot(int64_t m, int64_t n, double alpha, const double *A,
                        int64_t lda, double *B, int64_t ldb)
{
    int64_t i, j, k;
    if (m < 0 || n < 0 || lda < (m > 1 ? m : 1) || ldb < (m > 1 ? m : 1))
        return 1;
    for (j = 0; j < n; ++j) {
        double *b = B + j * ldb;
        if (alpha == 0.0) {
            for (i = 0; i < m; ++i) b[i] = 0.0;
            continue;
        }
        for (i = 0; i < m; ++i) {
            double s = alpha * b[i];
            for (k = 0; k < i; ++k) s = s - A[i + k * lda] * b[k];
            b[i] = s / A[i + i * lda];
        }
    }
    return 0;
}

/* ---- fp32 (computed in fp32, the operand precision) ------------------ */

static void solve_column_s(int64_t m, float alpha, const float *A,
                           int64_t lda, float *b)
{
    int64_t i, k;
    if (alpha == 0.0f) {
        for (i = 0; i < m; ++i) b[i] = 0.0f;
        return;
    }
    for (i = 0; i < m; ++i) b[i] = alpha * b[i];
    for (k = 0; k < m; ++k) {
        const float *lk = A + k * lda;
        float xk = b[k] / lk[k];
        b[k] = xk;
        for (i = k + 1; i < m; ++i) b[i] = b[i] - lk[i] * xk;
    }
}

int oracle_lln_s(int64_t m, int64_t n, float alpha, const float *A,
                 int64_t lda, float *B, int64_t ldb)
{
    int64_t j;
    if (m < 0 || n < 0 || lda < (m > 1 ? m : 1) || ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (j = 0; j < n; ++j) solve_column_s(m, alpha, A, lda, B + j * ldb);
    return 0;
}

/* ---- complex fp64, interleaved (re, im) ------------------------------ */

static void solve_column_z(int64_t m, double ar, double ai, const double *A,
                           int64_t lda, double *b)
{
    int64_t i, k;
    if (ar == 0.0 && ai == 0.0) {
        for (i = 0; i < 2 * m; ++i) b[i] = 0.0;
        return;
    }
    for (i = 0; i < m; ++i) {
        double br = b[2 * i], bi = b[2 * i + 1];
        b[2 * i]     = ar * br - ai * bi;
        b[2 * i + 1] = ar * bi + ai * br;
    }
    for (k = 0; k < m; ++k) {
        const double *lk = A + 2 * k * lda;
        double dr = lk[2 * k], di = lk[2 * k + 1];
        double br = b[2 * k], bi = b[2 * k + 1];
        double xr, xi;
        if (di == 0.0) {
            xr = br / dr;
            xi = bi / dr;
        } else {
            double den = dr * dr + di * di;
            xr = (br * dr + bi * di) / den;
            xi = (bi * dr - br * di) / den;
        }
        b[2 * k] = xr;
        b[2 * k + 1] = xi;
        for (i = k + 1; i < m; ++i) {
            double lr = lk[2 * i], li = lk[2 * i + 1];
            double pr = lr * xr - li * xi;
            double pi = lr * xi + li * xr;
            b[2 * i]     = b[2 * i] - pr;
            b[2 * i + 1] = b[2 * i + 1] - pi;
        }
    }
}

int oracle_lln_z(int64_t m, int64_t n, double alpha_re, double alpha_im,
                 const double *A, int64_t lda, double *B, int64_t ldb)
{
    int64_t j;
    if (m < 0 || n < 0 || lda < (m > 1 ? m : 1) || ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (j = 0; j < n; ++j)
        solve_column_z(m, alpha_re, alpha_im, A, lda, B + 2 * j * ldb);
    return 0;
}

/* ---- complex fp32, interleaved (re, im) floats ----------------------- */

static void solve_column_c(int64_t m, float ar, float ai, const float *A,
                           int64_t lda, float *b)
{
    int64_t i, k;
    if (ar == 0.0f && ai == 0.0f) {
        for (i = 0; i < 2 * m; ++i) b[i] = 0.0f;
        return;
    }
    for (i = 0; i < m; ++i) {
        float br = b[2 * i], bi = b[2 * i + 1];
        b[2 * i]     = ar * br - ai * bi;
        b[2 * i + 1] = ar * bi + ai * br;
    }
    for (k = 0; k < m; ++k) {
        const float *lk = A + 2 * k * lda;
        float dr = lk[2 * k], di = lk[2 * k + 1];
        float br = b[2 * k], bi = b[2 * k + 1];
        float xr, xi;
        if (di == 0.0f) {
            xr = br / dr;
            xi = bi / dr;
        } else {
            float den = dr * dr + di * di;
            xr = (br * dr + bi * di) / den;
            xi = (bi * dr - br * di) / den;
        }
        b[2 * k] = xr;
        b[2 * k + 1] = xi;
        for (i = k + 1; i < m; ++i) {
            float lr = lk[2 * i], li = lk[2 * i + 1];
            float pr = lr * xr - li * xi;
            float pi = lr * xi + li * xr;
            b[2 * i]     = b[2 * i] - pr;
            b[2 * i + 1] = b[2 * i + 1] - pi;
        }
    }
}

int oracle_lln_c(int64_t m, int64_t n, float alpha_re, float alpha_im,
                 const float *A, int64_t lda, float *B, int64_t ldb)
{
    int64_t j;
    if (m < 0 || n < 0 || lda < (m > 1 ? m : 1) || ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (j = 0; j < n; ++j)
        solve_column_c(m, alpha_re, alpha_im, A, lda, B + 2 * j * ldb);
    return 0;
}

/* ---- strided batches: problem p at A + p*strideA, B + p*strideB ------- */
/* Strides are in elements of the data type (complex elements for _z, _c). */

int oracle_lln_d_batched(int64_t m, int64_t n, double alpha, const double *A,
                         int64_t lda, int64_t strideA, double *B, int64_t ldb,
                         int64_t strideB, int64_t batch)
{
    int64_t p, j;
    if (m < 0 || n < 0 || batch < 0 || lda < (m > 1 ? m : 1) ||
        ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1) private(j)
    for (p = 0; p < batch; ++p)
        for (j = 0; j < n; ++j)
            solve_column_d(m, alpha, A + p * strideA, lda,
                           B + p * strideB + j * ldb);
    return 0;
}

int oracle_lln_s_batched(int64_t m, int64_t n, float alpha, const float *A,
                         int64_t lda, int64_t strideA, float *B, int64_t ldb,
                         int64_t strideB, int64_t batch)
{
    int64_t p, j;
    if (m < 0 || n < 0 || batch < 0 || lda < (m > 1 ? m : 1) ||
        ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1) private(j)
    for (p = 0; p < batch; ++p)
        for (j = 0; j < n; ++j)
            solve_column_s(m, alpha, A + p * strideA, lda,
                           B + p * strideB + j * ldb);
    return 0;
}

int oracle_lln_z_batched(int64_t m, int64_t n, double alpha_re,
                         double alpha_im, const double *A, int64_t lda,
                         int64_t strideA, double *B, int64_t ldb,
                         int64_t strideB, int64_t batch)
{
    int64_t p, j;
    if (m < 0 || n < 0 || batch < 0 || lda < (m > 1 ? m : 1) ||
        ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1) private(j)
    for (p = 0; p < batch; ++p)
        for (j = 0; j < n; ++j)
            solve_column_z(m, alpha_re, alpha_im, A + 2 * p * strideA, lda,
                           B + 2 * p * strideB + 2 * j * ldb);
    return 0;
}

int oracle_lln_c_batched(int64_t m, int64_t n, float alpha_re,
                         float alpha_im, const float *A, int64_t lda,
                         int64_t strideA, float *B, int64_t ldb,
                         int64_t strideB, int64_t batch)
{
    int64_t p, j;
    if (m < 0 || n < 0 || batch < 0 || lda < (m > 1 ? m : 1) ||
        ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1) private(j)
    for (p = 0; p < batch; ++p)
        for (j = 0; j < n; ++j)
            solve_column_c(m, alpha_re, alpha_im, A + 2 * p * strideA, lda,
                           B + 2 * p * strideB + 2 * j * ldb);
    return 0;
}

/* ---- every TRSM variant, by its definition ------------------------------
 *
 * The general BLAS TRSM (section 2.1 of the pages: op(A) X = alpha B, and its
 * right-side form X op(A) = alpha B):
 *   side  0: op(A) X = alpha B, A is m x m;  1: X op(A) = alpha B, A is n x n;
 *   uplo  0: the lower triangle of A is used, 1: the upper;
 *   trans 0: op(A) = A, 1: A^T, 2: A^H (conjugate transpose);
 *   diag  0: non-unit, 1: unit diagonal (the diagonal of A is not read);
 *   cplx  1: A and B hold interleaved complex values, 0: real values.
 * Each right-hand side -- a column of B for side 0, a row of B for side 1 --
 * is the solution y of a triangular system T y = alpha c, with T = op(A) for
 * side 0 and T = op(A)^T for side 1 (x op(A) = alpha b is, entry by entry,
 * sum_k x_k op(A)_kj = alpha b_j).  T is lower or upper triangular and is
 * solved by substitution starting where its triangle starts:
 *     y_i = (alpha c_i - sum_{j solved before i} T_ij y_j) / T_ii,
 * the solved terms subtracted in the order they were solved.  The complex
 * arithmetic is written out as above; real data run the same loops with
 * imaginary parts 0, which changes no rounding (every term with an
 * imaginary factor is an exact zero).
 */

/* Entry (i, k) of T, as (re, im). */
static void tget_d(int side, int trans, int cplx, const double *A, int64_t lda,
                   int64_t i, int64_t k, double *re, double *im)
{
    int64_t r = i, c = k;          /* entry (r, c) of op(A) */
    int64_t ar, ac;                /* entry (ar, ac) of A   */
    if (side == 1) { r = k; c = i; }
    if (trans == 0) { ar = r; ac = c; } else { ar = c; ac = r; }
    if (cplx) {
        *re = A[2 * (ar + ac * lda)];
        *im = A[2 * (ar + ac * lda) + 1];
        if (trans == 2) *im = -*im;
    } else {
        *re = A[ar + ac * lda];
        *im = 0.0;
    }
}

int oracle_trsm_d(int side, int uplo, int trans, int diag, int cplx, int64_t m,
                  int64_t n, double alpha_re, double alpha_im, const double *A,
                  int64_t lda, double *B, int64_t ldb)
{
    int64_t k = side == 0 ? m : n;       /* order of A and of T            */
    int64_t nrhs = side == 0 ? n : m;    /* number of right-hand sides     */
    int64_t cs = side == 0 ? 1 : ldb;    /* stride inside one right-hand side */
    int64_t rs = side == 0 ? ldb : 1;    /* stride between right-hand sides   */
    int e = cplx ? 2 : 1;
    int op_lower = (uplo == 0) == (trans == 0);
    int lower = side == 0 ? op_lower : !op_lower;
    int64_t q;
    if (side < 0 || side > 1 || uplo < 0 || uplo > 1 || trans < 0 || trans > 2 ||
        diag < 0 || diag > 1 || m < 0 || n < 0 || lda < (k > 1 ? k : 1) ||
        ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (q = 0; q < nrhs; ++q) {
        double *c = B + e * q * rs;
        int64_t t, u;
        if (alpha_re == 0.0 && alpha_im == 0.0) {
            for (t = 0; t < k; ++t) {
                c[e * t * cs] = 0.0;
                if (cplx) c[e * t * cs + 1] = 0.0;
            }
            continue;
        }
        for (t = 0; t < k; ++t) {
            int64_t i = lower ? t : k - 1 - t;
            double cr = c[e * i * cs], ci = cplx ? c[e * i * cs + 1] : 0.0;
            double sr = alpha_re * cr - alpha_im * ci;
            double si = alpha_re * ci + alpha_im * cr;
            for (u = 0; u < t; ++u) {
                int64_t j = lower ? u : k - 1 - u;
                double tr, ti;
                double yr = c[e * j * cs], yi = cplx ? c[e * j * cs + 1] : 0.0;
                tget_d(side, trans, cplx, A, lda, i, j, &tr, &ti);
                sr = sr - (tr * yr - ti * yi);
                si = si - (tr * yi + ti * yr);
            }
            if (!diag) {
                double dr, di;
                tget_d(side, trans, cplx, A, lda, i, i, &dr, &di);
                if (di == 0.0) {
                    sr = sr / dr;
                    si = si / dr;
                } else {
                    double den = dr * dr + di * di;
                    double xr = (sr * dr + si * di) / den;
                    double xi = (si * dr - sr * di) / den;
                    sr = xr;
                    si = xi;
                }
            }
            c[e * i * cs] = sr;
            if (cplx) c[e * i * cs + 1] = si;
        }
    }
    return 0;
}

/* The same in fp32 (the operand precision of fp32 and complex fp32). */

static void tget_s(int side, int trans, int cplx, const float *A, int64_t lda,
                   int64_t i, int64_t k, float *re, float *im)
{
    int64_t r = i, c = k;          /* entry (r, c) of op(A) */
    int64_t ar, ac;                /* entry (ar, ac) of A   */
    if (side == 1) { r = k; c = i; }
    if (trans == 0) { ar = r; ac = c; } else { ar = c; ac = r; }
    if (cplx) {
        *re = A[2 * (ar + ac * lda)];
        *im = A[2 * (ar + ac * lda) + 1];
        if (trans == 2) *im = -*im;
    } else {
        *re = A[ar + ac * lda];
        *im = 0.0f;
    }
}

int oracle_trsm_s(int side, int uplo, int trans, int diag, int cplx, int64_t m,
                  int64_t n, float alpha_re, float alpha_im, const float *A,
                  int64_t lda, float *B, int64_t ldb)
{
    int64_t k = side == 0 ? m : n;       /* order of A and of T            */
    int64_t nrhs = side == 0 ? n : m;    /* number of right-hand sides     */
    int64_t cs = side == 0 ? 1 : ldb;    /* stride inside one right-hand side */
    int64_t rs = side == 0 ? ldb : 1;    /* stride between right-hand sides   */
    int e = cplx ? 2 : 1;
    int op_lower = (uplo == 0) == (trans == 0);
    int lower = side == 0 ? op_lower : !op_lower;
    int64_t q;
    if (side < 0 || side > 1 || uplo < 0 || uplo > 1 || trans < 0 || trans > 2 ||
        diag < 0 || diag > 1 || m < 0 || n < 0 || lda < (k > 1 ? k : 1) ||
        ldb < (m > 1 ? m : 1))
        return 1;
    #pragma omp parallel for schedule(dynamic, 1)
    for (q = 0; q < nrhs; ++q) {
        float *c = B + e * q * rs;
        int64_t t, u;
        if (alpha_re == 0.0f && alpha_im == 0.0f) {
            for (t = 0; t < k; ++t) {
                c[e * t * cs] = 0.0f;
                if (cplx) c[e * t * cs + 1] = 0.0f;
            }
            continue;
        }
        for (t = 0; t < k; ++t) {
            int64_t i = lower ? t : k - 1 - t;
            float cr = c[e * i * cs], ci = cplx ? c[e * i * cs + 1] : 0.0f;
            float sr = alpha_re * cr - alpha_im * ci;
            float si = alpha_re * ci + alpha_im * cr;
            for (u = 0; u < t; ++u) {
                int64_t j = lower ? u : k - 1 - u;
                float tr, ti;
                float yr = c[e * j * cs], yi = cplx ? c[e * j * cs + 1] : 0.0f;
                tget_s(side, trans, cplx, A, lda, i, j, &tr, &ti);
                sr = sr - (tr * yr - ti * yi);
                si = si - (tr * yi + ti * yr);
            }
            if (!diag) {
                float dr, di;
                tget_s(side, trans, cplx, A, lda, i, i, &dr, &di);
                if (di == 0.0f) {
                    sr = sr / dr;
                    si = si / dr;
                } else {
                    float den = dr * dr + di * di;
                    float xr = (sr * dr + si * di) / den;
                    float xi = (si * dr - sr * di) / den;
                    sr = xr;
                    si = xi;
                }
            }
            c[e * i * cs] = sr;
            if (cplx) c[e * i * cs + 1] = si;
        }
    }
    return 0;
}

/* Number of OpenMP threads a parallel region here would use. */
int oracle_num_threads(void)
{
    int t = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
