// Kernel (a): direct solve of L X = alpha B for m <= 64 in one workgroup.
//
// Follows the small-regime design of HSMA-TRSM ("Hierarchical Shared
// Memory-Aware Optimization for TRSM on GPU Platforms", section 4.2.1 and
// Figure 3): the triangle of L is staged on chip, each thread keeps one
// right-hand-side column in registers, and solved rows update the rows below
// them.  The loops are fully unrolled so the column lives in registers with
// compile-time indices (section 4.2.1, "Compute-Memory Overlap").
//
// gfx950 mapping:
//   * one workgroup per (problem, group of 64 columns); lane j of every wave
//     owns column j of the group;
//   * the m <= 64 rows are cut into W = ceil(m/16) panels of 16 rows; wave w
//     owns panel w of every column (16 values per lane in VGPRs);
//   * L's lower 16x16 blocks are packed in LDS (W(W+1)/2 blocks; 40 KB for
//     complex fp64 at m = 64, so two workgroups fit in the 160 KB LDS of a CU
//     next to the panel exchange buffers);
//   * step p: wave p solves its diagonal block in registers (L from LDS,
//     read at one address per wave, i.e. broadcast), publishes the 16 solved
//     rows through a double-buffered LDS panel and stores them to HBM; after
//     one barrier every wave q > p subtracts L[q-block, p-block] * X_p.
// The 64 KB per-block limits that forced the pages' dual thread-group
// pipeline for complex fp64 (section 4.2.2) do not exist here: the whole
// problem fits in one CU's LDS and VGPRs.
#include "scalar_ops.h"

namespace trsm {
namespace {

constexpr int kPanel = 16;  // rows per wave panel
constexpr int kCols = 64;   // right-hand-side columns per workgroup (one per lane)

template <typename T, int W>
__global__ __launch_bounds__(64 * W, 2) void small_lln_kernel(int m, int64_t n, int64_t ncg,
                                                          Scalar alpha_s, const T *__restrict__ A,
                                                          int64_t lda, int64_t strideA,
                                                          T *__restrict__ B, int64_t ldb,
                                                          int64_t strideB) {
    using E = Elem<T>;
    constexpr int kBlocks = W * (W + 1) / 2;
    __shared__ T Ls[kBlocks][kPanel * kPanel];  // block (bw, bp) at bw(bw+1)/2 + bp, col-major
    __shared__ T invd[W * kPanel];
    __shared__ T Xs[2][kPanel][kCols];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t prob = blockIdx.x / ncg;
    const int64_t cg = blockIdx.x - prob * ncg;
    const T *__restrict__ Ap = A + prob * strideA;
    T *__restrict__ Bp = B + prob * strideB;
    const int64_t j = cg * kCols + lane;
    const bool colok = j < n;
    const T alpha = E::from(alpha_s);

    // Stage the lower blocks of L (zeros outside the triangle and beyond m,
    // so padded rows solve to exact zeros and are never stored).
    for (int idx = threadIdx.x; idx < kBlocks * kPanel * kPanel; idx += 64 * W) {
        const int blk = idx / (kPanel * kPanel);
        const int e = idx - blk * kPanel * kPanel;
        int bw = 0;
        while ((bw + 1) * (bw + 2) / 2 <= blk) ++bw;
        const int bp = blk - bw * (bw + 1) / 2;
        const int i = bw * kPanel + (e % kPanel);
        const int k = bp * kPanel + (e / kPanel);
        T v = E::zero();
        if (i < m && k < m && i >= k) v = Ap[i + (int64_t)k * lda];
        Ls[blk][e] = v;
    }
    for (int i = threadIdx.x; i < W * kPanel; i += 64 * W)
        invd[i] = (i < m) ? E::recip(Ap[i + (int64_t)i * lda]) : E::zero();

    // This wave's 16 rows of column j, scaled by alpha.
    T b[kPanel];
#pragma unroll
    for (int r = 0; r < kPanel; ++r) {
        const int i = w * kPanel + r;
        b[r] = (colok && i < m) ? E::mul(alpha, Bp[i + j * ldb]) : E::zero();
    }
    __syncthreads();

#pragma unroll
    for (int p = 0; p < W; ++p) {
        if (w == p) {
            const T *Ld = Ls[p * (p + 1) / 2 + p];
#pragma unroll
            for (int k = 0; k < kPanel; ++k) {
                const T xk = E::mul(b[k], invd[p * kPanel + k]);
                b[k] = xk;
#pragma unroll
                for (int r = k + 1; r < kPanel; ++r) b[r] = E::msub(b[r], Ld[k * kPanel + r], xk);
            }
#pragma unroll
            for (int r = 0; r < kPanel; ++r) Xs[p & 1][r][lane] = b[r];
#pragma unroll
            for (int r = 0; r < kPanel; ++r) {
                const int i = p * kPanel + r;
                if (colok && i < m) Bp[i + j * ldb] = b[r];
            }
        }
        __syncthreads();
        if (w > p) {
            const T *Lo = Ls[w * (w + 1) / 2 + p];
#pragma unroll
            for (int k = 0; k < kPanel; ++k) {
                const T xk = Xs[p & 1][k][lane];
#pragma unroll
                for (int r = 0; r < kPanel; ++r) b[r] = E::msub(b[r], Lo[k * kPanel + r], xk);
            }
        }
    }
}

template <typename T>
hipError_t launch_t(int m, int64_t n, Scalar alpha, const void *A, int64_t lda, int64_t sA,
                    void *B, int64_t ldb, int64_t sB, int64_t batch, hipStream_t st) {
    const int64_t ncg = (n + kCols - 1) / kCols;
    const int64_t nblk = ncg * batch;
    if (nblk <= 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int W = (m + kPanel - 1) / kPanel;
    const T *a = static_cast<const T *>(A);
    T *b = static_cast<T *>(B);
    dim3 grid((unsigned)nblk);
    switch (W) {
        case 1: hipLaunchKernelGGL((small_lln_kernel<T, 1>), grid, dim3(64), 0, st, m, n, ncg, alpha, a, lda, sA, b, ldb, sB); break;
        case 2: hipLaunchKernelGGL((small_lln_kernel<T, 2>), grid, dim3(128), 0, st, m, n, ncg, alpha, a, lda, sA, b, ldb, sB); break;
        case 3: hipLaunchKernelGGL((small_lln_kernel<T, 3>), grid, dim3(192), 0, st, m, n, ncg, alpha, a, lda, sA, b, ldb, sB); break;
        case 4: hipLaunchKernelGGL((small_lln_kernel<T, 4>), grid, dim3(256), 0, st, m, n, ncg, alpha, a, lda, sA, b, ldb, sB); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t small_lln_launch(int dtype, int m, int64_t n, Scalar alpha, const void *A,
                            int64_t lda, int64_t strideA, void *B, int64_t ldb,
                            int64_t strideB, int64_t batch, hipStream_t stream) {
    if (m < 1 || m > 64) return hipErrorInvalidValue;
    // fp64 and complex fp64 run on the matrix cores (small_mfma.hip); fp32
    // and complex fp32 on the vector units here.
    if (dtype == R64F || dtype == C64F)
        return small_mfma_launch(dtype, m, n, alpha, A, lda, strideA, B, ldb, strideB, batch,
                                 stream);
    switch (dtype) {
        case R32F: return launch_t<float>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch, stream);
        case R64F: return launch_t<double>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch, stream);
        case C64F: return launch_t<cplx>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch, stream);
        case C32F: return launch_t<cplx32>(m, n, alpha, A, lda, strideA, B, ldb, strideB, batch, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace trsm
