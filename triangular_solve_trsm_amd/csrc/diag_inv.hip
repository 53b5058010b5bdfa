// Kernel (b1): inversion of the diagonal blocks of L (phase 1 of the blocked
// algorithm).
//
// HSMA-TRSM ("Hierarchical Shared Memory-Aware Optimization for TRSM on GPU
// Platforms"), section 4.3 "Phase 1" and section 4.3.1 with Figures 6 and 7:
// the ceil(m/ib) diagonal blocks D_t are independent and are inverted in
// parallel; each inverse is produced by plain substitution against columns of
// the identity (the tile E_j), streaming one column of D_t at a time, so the
// on-chip footprint grows with ib and not with ib^2; the next column is
// fetched while the current one is used (double buffering).
//
// gfx950 mapping (one wavefront per workgroup, no barriers):
//   * workgroup (t, c) computes columns [c*P, c*P + P) of W_t = D_t^{-1};
//   * lane l owns rows l*R .. l*R + R - 1 (R = ib/64) of those P columns, as
//     R x P values in VGPRs (the identity tile is generated in registers);
//   * step k (k = c*P .. bs-1): the lane owning row k scales its row by the
//     reciprocal of d_kk; the P solved values are broadcast to the wave with
//     v_readlane (SGPR operands of the following FMAs); every lane subtracts
//     d_ik * x_k from its rows i > k;
//   * column k of D_t is read straight into VGPRs, each lane its own rows,
//     and column k+1 is prefetched into a second register set while column k
//     is used -- the two-buffer alternation of Figure 7, held in registers
//     (the CDNA4 register file is 512 KB per CU) instead of shared memory;
//     LDS is not used at all, so the footprint is O(ib) per wavefront.
// Rows above the diagonal are written as explicit zeros, which the triangular
// GEMM of the solve phase relies on.
#include "scalar_ops.h"

namespace trsm {
namespace {

__device__ __forceinline__ float bcast(float v, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
__device__ __forceinline__ double bcast(double v, int src) {
    const long long bits = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_readlane((int)(bits & 0xffffffffLL), src);
    const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), src);
    const unsigned long long r =
        ((unsigned long long)(unsigned)hi << 32) | (unsigned long long)(unsigned)lo;
    return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ cplx bcast(cplx v, int src) {
    return cplx{bcast(v.re, src), bcast(v.im, src)};
}

template <typename T> constexpr int words() { return sizeof(T) / 4; }

// Columns per wavefront: keep R x P values of T within 128 VGPRs.
template <typename T, int R>
constexpr int panel_cols() {
    constexpr int ib = 64 * R;
    constexpr int p = 128 / (R * words<T>());
    return p < ib ? p : ib;
}

template <typename T, int R>
__global__ __launch_bounds__(64) void diag_inv_kernel(int64_t m, const T *__restrict__ A,
                                                      int64_t lda, T *__restrict__ W,
                                                      int npanels) {
    using E = Elem<T>;
    constexpr int IB = 64 * R;
    constexpr int P = panel_cols<T, R>();
    const int t = blockIdx.x / npanels;
    const int c = blockIdx.x - t * npanels;
    const int lane = threadIdx.x;
    const int64_t base = (int64_t)t * IB;
    const int bs = (int)((m - base) < IB ? (m - base) : IB);
    const int j0 = c * P;
    if (j0 >= bs) return;
    const T *__restrict__ D = A + base + base * lda;  // D(i, k) = D[i + k*lda]
    T *__restrict__ Wt = W + (int64_t)t * IB * IB;

    // identity tile E_j for columns j0 .. j0+P-1, and reciprocals of own pivots
    T x[R][P];
    T inv[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int i = lane * R + rr;
        inv[rr] = (i < bs) ? E::recip(D[i + (int64_t)i * lda]) : E::zero();
#pragma unroll
        for (int jj = 0; jj < P; ++jj) x[rr][jj] = (i == j0 + jj) ? E::one() : E::zero();
    }

    // column k of D for own rows i > k (strict lower part only)
    auto load_col = [&](int k, T *dst) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int i = lane * R + rr;
            dst[rr] = (k < bs && i > k && i < bs) ? D[i + (int64_t)k * lda] : E::zero();
        }
    };

    T dnext[R];
    load_col(j0, dnext);
    const int kb_first = j0 / R;
    const int kb_last = (bs - 1) / R;
    for (int kb = kb_first; kb <= kb_last; ++kb) {  // kb = lane owning rows kb*R ..
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int k = kb * R + r;
            if (k < j0) continue;  // wave-uniform
            if (k >= bs) break;    // wave-uniform
            T dcur[R];
#pragma unroll
            for (int rr = 0; rr < R; ++rr) dcur[rr] = dnext[rr];
            load_col(k + 1, dnext);  // prefetch the next column
            T s[P];
#pragma unroll
            for (int jj = 0; jj < P; ++jj) s[jj] = bcast(E::mul(x[r][jj], inv[r]), kb);
#pragma unroll
            for (int rr = 0; rr < R; ++rr) {
                const int i = lane * R + rr;
                if (i == k) {
#pragma unroll
                    for (int jj = 0; jj < P; ++jj) x[rr][jj] = s[jj];
                } else if (i > k) {
#pragma unroll
                    for (int jj = 0; jj < P; ++jj) x[rr][jj] = E::msub(x[rr][jj], dcur[rr], s[jj]);
                }
            }
        }
    }

#pragma unroll
    for (int jj = 0; jj < P; ++jj) {
        const int j = j0 + jj;
        if (j >= bs) break;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int i = lane * R + rr;
            if (i < bs) Wt[i + (int64_t)j * IB] = x[rr][jj];
        }
    }
}

template <typename T, int R>
hipError_t launch_r(int64_t m, const void *A, int64_t lda, void *W, hipStream_t st) {
    constexpr int IB = 64 * R;
    constexpr int P = panel_cols<T, R>();
    const int64_t nb = (m + IB - 1) / IB;
    const int npanels = (IB + P - 1) / P;
    const int64_t grid = nb * npanels;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((diag_inv_kernel<T, R>), dim3((unsigned)grid), dim3(64), 0, st, m,
                       static_cast<const T *>(A), lda, static_cast<T *>(W), npanels);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(int ib, int64_t m, const void *A, int64_t lda, void *W, hipStream_t st) {
    switch (ib) {
        case 64: return launch_r<T, 1>(m, A, lda, W, st);
        case 128: return launch_r<T, 2>(m, A, lda, W, st);
        case 256: return launch_r<T, 4>(m, A, lda, W, st);
        case 512: return launch_r<T, 8>(m, A, lda, W, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t diag_inv_launch(int dtype, int ib, int64_t m, const void *A, int64_t lda, void *W,
                           hipStream_t stream) {
    switch (dtype) {
        case R32F: return launch_t<float>(ib, m, A, lda, W, stream);
        case R64F: return launch_t<double>(ib, m, A, lda, W, stream);
        case C64F: return launch_t<cplx>(ib, m, A, lda, W, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace trsm
