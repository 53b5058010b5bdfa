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
//   * task (t, c) computes columns [c*P, c*P + P) of W_t = D_t^{-1}; the
//     tasks of one block run on one XCD, sharing its L2;
//   * lane l owns rows l*R .. l*R + R - 1 (R = ib/64) of those P columns, as
//     R x P values in VGPRs (the identity tile is generated in registers);
//   * step k (k = c*P .. bs-1): the lane owning row k scales its row by the
//     reciprocal of d_kk; the P solved values are broadcast to the wave with
//     v_readlane (SGPR operands of the following FMAs); every lane subtracts
//     d_ik * x_k from its rows i > k;
//   * column k of D_t is read straight into VGPRs, each lane its own rows.
//     Figure 7 alternates two column buffers (compute one, fetch the next);
//     here the buffers are a ring of several columns in registers (the CDNA4
//     register file is 512 KB per CU), because one column ahead is far less
//     than the memory latency at a few hundred cycles per step.  LDS is not
//     used at all, so the footprint stays O(ib) per wavefront.
// Rows above the diagonal are written as explicit zeros, which the triangular
// GEMM of the solve phase relies on.
#include "buffer_ops.h"
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

// Columns of D in flight: a ring of DP columns (R values of T per lane each)
// within 128 VGPRs, between 2 and 16.  At a few hundred cycles per step,
// several columns ahead cover the memory latency that one column ahead left
// exposed on every step.
template <typename T, int R>
constexpr int ring_cols() {
    constexpr int d = 128 / (R * words<T>());
    return d < 2 ? 2 : (d > 16 ? 16 : d);
}

template <typename T, int R, bool VEC>
__global__ __launch_bounds__(64) void diag_inv_kernel(int64_t m, const T *__restrict__ A,
                                                      int64_t lda, T *__restrict__ W,
                                                      int npanels) {
    using E = Elem<T>;
    constexpr int IB = 64 * R;
    constexpr int P = panel_cols<T, R>();
    constexpr int DP = ring_cols<T, R>();
    constexpr int U = DP > R ? DP : R;  // steps per unrolled group (multiple of both)
    // Workgroups go round-robin to the 8 XCDs (workgroup b on XCD b % 8);
    // give each XCD a contiguous run of (block, panel) tasks so that the
    // waves reading one diagonal block share that XCD's L2.
    const int total = (int)((m + IB - 1) / IB) * npanels;
    const int per = (total + 7) / 8;
    const int q = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (q >= total) return;
    const int t = q / npanels;
    const int c = q - t * npanels;
    const int lane = threadIdx.x;
    const int64_t base = (int64_t)t * IB;
    const int bs = (int)((m - base) < IB ? (m - base) : IB);
    const int j0 = c * P;
    if (j0 >= bs) return;
    T *__restrict__ Wt = W + (int64_t)t * IB * IB;
    // D(i, k) at element i + k * lda from here; reads past A's last element
    // return zero (they only reach rows and columns >= bs, which are unused).
    const int64_t doff = base + base * lda;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(A + doff, ((m - 1) + (m - 1) * lda + 1 - doff) * (int64_t)sizeof(T));
    const int row0 = lane * R;  // this lane's rows row0 .. row0 + R - 1
    auto col_off = [&](int k) -> uint32_t {
        return (uint32_t)(((int64_t)row0 + (int64_t)k * lda) * (int64_t)sizeof(T));
    };

    // identity tile E_j for columns j0 .. j0+P-1, and reciprocals of own pivots
    T x[R][P];
    T inv[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int i = row0 + rr;
        T d[1];
        ld_elems<T, 1, false>(rs, (uint32_t)(((int64_t)i + (int64_t)i * lda) * (int64_t)sizeof(T)), d);
        inv[rr] = E::recip(d[0]);
#pragma unroll
        for (int jj = 0; jj < P; ++jj) x[rr][jj] = E::sel(i == j0 + jj, E::one(), E::zero());
    }

    // Steps run in groups of U starting at a multiple of U, so that the
    // pivot row inside its lane (k % R) and the ring slot (k % DP) are
    // compile-time indices; steps before j0 are skipped.  Column loads are
    // unconditional, so the compiler can keep DP of them in flight.
    const int k_begin = (j0 / U) * U;
    T ring[DP][R];
#pragma unroll
    for (int u = 0; u < DP; ++u) ld_elems<T, R, VEC>(rs, col_off(k_begin + u), ring[u]);
    for (int k0 = k_begin; k0 < bs; k0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + u;
            const int slot = u % DP;
            const int r = u % R;
            if (k >= j0 && k < bs) {  // wave-uniform
                const int kb = k / R;  // lane owning row k
                T s[P];
#pragma unroll
                for (int jj = 0; jj < P; ++jj) s[jj] = bcast(E::mul(x[r][jj], inv[r]), kb);
                // rows below the pivot: x_i -= d_ik s (d masked to 0 for i <= k)
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    const T d = E::sel(row0 + rr > k, ring[slot][rr], E::zero());
#pragma unroll
                    for (int jj = 0; jj < P; ++jj) x[rr][jj] = E::msub(x[rr][jj], d, s[jj]);
                }
                // the pivot row itself takes the solved values
                const bool own = lane == kb;
#pragma unroll
                for (int jj = 0; jj < P; ++jj) x[r][jj] = E::sel(own, s[jj], x[r][jj]);
            }
            ld_elems<T, R, VEC>(rs, col_off(k + DP), ring[slot]);  // refill the slot just used
        }
    }

#pragma unroll
    for (int jj = 0; jj < P; ++jj) {
        const int j = j0 + jj;
        if (j >= bs) break;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int i = row0 + rr;
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
    const int64_t total = nb * npanels;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL - 8) return hipErrorInvalidConfiguration;
    const int64_t grid = 8 * ((total + 7) / 8);  // whole rounds over the 8 XCDs
    // 32-bit buffer offsets reach one diagonal block: IB columns of lda
    if ((int64_t)sizeof(T) * (lda + 1) * IB > 0x7fffffffLL) return hipErrorInvalidValue;
    const int vec = (reinterpret_cast<uintptr_t>(A) % 16 == 0) &&
                    ((int64_t)sizeof(T) * lda) % 16 == 0;
    if (vec)
        hipLaunchKernelGGL((diag_inv_kernel<T, R, true>), dim3((unsigned)grid), dim3(64), 0, st, m,
                           static_cast<const T *>(A), lda, static_cast<T *>(W), npanels);
    else
        hipLaunchKernelGGL((diag_inv_kernel<T, R, false>), dim3((unsigned)grid), dim3(64), 0, st, m,
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
