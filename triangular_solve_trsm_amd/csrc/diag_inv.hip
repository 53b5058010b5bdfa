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
// On gfx950 the substitution is a serial chain as long as the block: at
// ib = 512 the wave that owns the first columns runs 512 dependent steps
// while the chip holds few enough tasks to leave most SIMDs idle.  So the
// substitution is used at 64 x 64 only, and the rest is built by recursive
// doubling on the matrix cores:
//
//   1. every 64 x 64 diagonal block is inverted by the column-streamed
//      substitution below, written straight into its place in W;
//   2. for b = 64, 128, .., ib/2 each pair of neighbouring inverted b x b
//      blocks [W11 0; . W22] of one ib block becomes the inverse of the
//      2b x 2b block [L11 0; L21 L22] through its lower-left block
//      X21 = -W22 L21 W11, two batched GEMMs per level (W22 L21 with the
//      triangular A path, then -(W22 L21) W11 with the triangular Bm path:
//      both skip the zero half of their triangular factor).
//
// Substitution kernel, gfx950 mapping (one wavefront per workgroup, no
// barriers):
//   * task (t, c) computes columns [c*P, c*P + P) of the inverse of 64R x 64R
//     diagonal block t; the tasks of one block run on one XCD, sharing its L2;
//   * lane l owns rows l*R .. l*R + R - 1 of those P columns, as R x P values
//     in VGPRs (the identity tile is generated in registers);
//   * step k (k = c*P .. bs-1): the lane owning row k scales its row by the
//     reciprocal of d_kk; the P solved values are broadcast to the wave with
//     v_readlane (SGPR operands of the following FMAs); every lane subtracts
//     d_ik * x_k from its rows i > k;
//   * column k of D_t is read straight into VGPRs, each lane its own rows.
//     Figure 7 alternates two column buffers (compute one, fetch the next);
//     here the buffers are a ring of several columns in registers, because
//     one column ahead is far less than the memory latency.  LDS is not used.
// Everything above the diagonal of each ib x ib block of W is written as an
// explicit zero (the substitution tile's own upper part, and the columns
// right of it inside the ib block): the doubling step's products and the
// triangular GEMM of the solve phase skip only whole zero K tiles and rely
// on the zeros inside the tiles they do read.
#include <cstdlib>
#include <cstring>

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
__device__ __forceinline__ cplx32 bcast(cplx32 v, int src) {
    return cplx32{bcast(v.re, src), bcast(v.im, src)};
}

template <typename T> constexpr int words() { return sizeof(T) / 4; }

// Columns of D in flight: a ring of DP columns (R values of T per lane each)
// within 128 VGPRs, between 2 and 16.  At a few hundred cycles per step,
// several columns ahead cover the memory latency that one column ahead left
// exposed on every step.
template <typename T, int R>
constexpr int ring_cols() {
    constexpr int d = 128 / (R * words<T>());
    return d < 2 ? 2 : (d > 16 ? 16 : d);
}

// Diagonal blocks of 64R x 64R, P columns per task.  Block t (rows
// [t*64R, ..)) is written at its place inside the ldw x ldw blocks of W
// (ldw a multiple of 64R): parent block t*64R / ldw, at rows and columns
// (t*64R) % ldw of it.
// WIDE: lda is so large that the 64R columns of one diagonal block span
// more than a 32-bit buffer offset reaches; each column of D then gets a
// buffer resource of its own (its base is wave-uniform, so this is scalar
// work), and the pivots are read with 64-bit addresses.
template <typename T, int R, int P, bool VEC, bool WIDE>
__global__ __launch_bounds__(64) void diag_inv_kernel(int64_t m, const T *__restrict__ A,
                                                      int64_t lda, T *__restrict__ W, int ldw,
                                                      int npanels) {
    using E = Elem<T>;
    constexpr int IB = 64 * R;
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
    const int row0 = lane * R;  // this lane's rows row0 .. row0 + R - 1
    const int64_t tp = base / ldw;
    const int lo = (int)(base - tp * ldw);
    const int bsp = (int)((m - tp * ldw) < ldw ? (m - tp * ldw) : ldw);
    T *__restrict__ Wt = W + tp * (int64_t)ldw * ldw + (int64_t)lo * (ldw + 1);
    // zeros in this block's rows right of it inside the parent block, the
    // columns shared out over the panel tasks
    for (int j = IB + c; lo + j < bsp; j += npanels) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
            if (row0 + rr < bs) Wt[row0 + rr + (int64_t)j * ldw] = E::zero();
    }
    const int j0 = c * P;
    if (j0 >= bs) return;
    // D(i, k) at element i + k * lda from here; reads past A's last element
    // return zero (they only reach rows and columns >= bs, which are unused).
    const int64_t doff = base + base * lda;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(A + doff, WIDE ? 0 : ((m - 1) + (m - 1) * lda + 1 - doff) * (int64_t)sizeof(T));
    // rows row0 .. row0+R-1 of column k of D; past the block they read zero
    auto load_col = [&](int k, T (&dst)[R]) {
        if constexpr (WIDE) {
            const __amdgpu_buffer_rsrc_t rc =
                make_rsrc(A + doff + (int64_t)k * lda, k < bs ? (int64_t)bs * (int64_t)sizeof(T) : 0);
            ld_elems<T, R, VEC>(rc, (uint32_t)(row0 * (int)sizeof(T)), dst);
        } else {
            ld_elems<T, R, VEC>(rs, (uint32_t)(((int64_t)row0 + (int64_t)k * lda) * (int64_t)sizeof(T)), dst);
        }
    };

    // identity tile E_j for columns j0 .. j0+P-1, and reciprocals of own pivots
    T x[R][P];
    T inv[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        const int i = row0 + rr;
        T d[1];
        if constexpr (WIDE)
            d[0] = i < bs ? A[doff + (int64_t)i + (int64_t)i * lda] : E::one();
        else
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
    for (int u = 0; u < DP; ++u) load_col(k_begin + u, ring[u]);
    for (int k0 = k_begin; k0 < bs; k0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + u;
            const int slot = u % DP;
            const int r = u % R;
            if (k >= j0 && k < bs) {  // wave-uniform
                const int kb = k / R;  // lane owning row k
                // Column j of the inverse is solved from step j on; before
                // that its row k is zero, and its solved value is zero too
                // (not 0 * (1/d_kk), which is NaN when d_kk is 0: such a NaN
                // would land above the diagonal, where W must hold zeros).
                // Only the task's first P - 1 steps have columns that are not
                // yet active (a uniform test).
                T s[P];
                if (k >= j0 + P - 1) {
#pragma unroll
                    for (int jj = 0; jj < P; ++jj) s[jj] = bcast(E::mul(x[r][jj], inv[r]), kb);
                } else {
#pragma unroll
                    for (int jj = 0; jj < P; ++jj)
                        s[jj] = bcast(E::sel(j0 + jj <= k, E::mul(x[r][jj], inv[r]), E::zero()), kb);
                }
                // rows below the pivot: x_i -= d_ik s.  Rows i <= k are left
                // as they are (a zero d would still turn an infinite s into
                // NaN there); the condition is per lane, so the update is
                // masked rather than selected element by element.
#pragma unroll
                for (int rr = 0; rr < R; ++rr) {
                    if (row0 + rr > k) {
                        const T d = ring[slot][rr];
#pragma unroll
                        for (int jj = 0; jj < P; ++jj) x[rr][jj] = E::msub(x[rr][jj], d, s[jj]);
                    }
                }
                // the pivot row itself takes the solved values
                const bool own = lane == kb;
#pragma unroll
                for (int jj = 0; jj < P; ++jj) x[r][jj] = E::sel(own, s[jj], x[r][jj]);
            }
            load_col(k + DP, ring[slot]);  // refill the slot just used
        }
    }

#pragma unroll
    for (int jj = 0; jj < P; ++jj) {
        const int j = j0 + jj;
        if (j >= bs) break;
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int i = row0 + rr;
            if (i < bs) Wt[i + (int64_t)j * ldw] = x[rr][jj];
        }
    }
}

template <typename T, int R, int P>
hipError_t launch_r(int64_t m, const void *A, int64_t lda, void *W, int ldw, hipStream_t st) {
    constexpr int IB = 64 * R;
    const int64_t nb = (m + IB - 1) / IB;
    const int npanels = (IB + P - 1) / P;
    const int64_t total = nb * npanels;
    if (total <= 0) return hipSuccess;
    if (total > 0x7fffffffLL - 8) return hipErrorInvalidConfiguration;
    if (ldw % IB != 0) return hipErrorInvalidValue;
    const int64_t grid = 8 * ((total + 7) / 8);  // whole rounds over the 8 XCDs
    // one buffer resource reaches a whole diagonal block (IB columns of lda)
    // while that spans less than 2 GB; beyond, one resource per column
    const bool wide = (int64_t)sizeof(T) * (lda + 1) * IB > 0x7fffffffLL;
    const int vec = (reinterpret_cast<uintptr_t>(A) % 16 == 0) &&
                    ((int64_t)sizeof(T) * lda) % 16 == 0;
    const T *a = static_cast<const T *>(A);
    T *w = static_cast<T *>(W);
    const dim3 g((unsigned)grid);
    if (wide && vec)
        hipLaunchKernelGGL((diag_inv_kernel<T, R, P, true, true>), g, dim3(64), 0, st, m, a, lda, w, ldw, npanels);
    else if (wide)
        hipLaunchKernelGGL((diag_inv_kernel<T, R, P, false, true>), g, dim3(64), 0, st, m, a, lda, w, ldw, npanels);
    else if (vec)
        hipLaunchKernelGGL((diag_inv_kernel<T, R, P, true, false>), g, dim3(64), 0, st, m, a, lda, w, ldw, npanels);
    else
        hipLaunchKernelGGL((diag_inv_kernel<T, R, P, false, false>), g, dim3(64), 0, st, m, a, lda, w, ldw, npanels);
    return hipGetLastError();
}

// 64 x 64 substitution with 8 columns per task: eight tasks per block keep
// the chain short (64 steps of 8 broadcasts and 8 FMAs each) and give the
// chip m/8 waves (16 columns per task measured 23.5 us for fp32 4096^2,
// 8 columns 16.0 us).
constexpr int kBase = 64;
constexpr int kBaseCols = 8;

hipError_t launch_base(int dtype, int64_t m, const void *A, int64_t lda, void *W, int ldw,
                       hipStream_t st) {
    switch (dtype) {
        case R32F: return launch_r<float, 1, kBaseCols>(m, A, lda, W, ldw, st);
        case R64F: return launch_r<double, 1, kBaseCols>(m, A, lda, W, ldw, st);
        case C64F: return launch_r<cplx, 1, kBaseCols>(m, A, lda, W, ldw, st);
        case C32F: return launch_r<cplx32, 1, kBaseCols>(m, A, lda, W, ldw, st);
        default: return hipErrorInvalidValue;
    }
}

// ---- fused base: whole NB x NB diagonal blocks in LDS ----------------------
// One workgroup (four waves) inverts one NB x NB diagonal block (NB = 128,
// or 64 for complex fp64, whose 128-block would not fit in LDS):
//   1. the block's lower triangle is loaded into LDS (zeros above the
//      diagonal, identity past the end of L);
//   2. its 16 x 16 diagonal blocks are inverted by substitution, one lane
//      per column (16 steps, each a short dot product with the solved rows);
//   3. recursive doubling 16 -> 32 -> .. -> NB inside LDS, X21 = -W22 L21 W11
//      for every pair of neighbouring blocks, both products on the matrix
//      cores (16 x 16 output tiles over the four waves, the zero half of the
//      triangular factor skipped); the product W22 L21 is kept in the pair's
//      upper-right quadrant, which is zero in the result and is cleared
//      again after use;
//   4. the block is written to W.
// So the 64 x 64 substitution and the first doubling level (two batched
// launches) become one launch whose serial chain is 16 steps long.
// Workgroups past the blocks write the zeros right of each block inside its
// ib x ib parent, 64 columns each, alongside.
template <typename T> struct InvMma;
template <> struct InvMma<float> {
    typedef float v4 __attribute__((ext_vector_type(4)));
    struct Acc { v4 a; };
    __device__ __forceinline__ static void zero(Acc &c) { c.a = v4{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ static void mma(float x, float y, Acc &c) {
        c.a = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c.a, 0, 0, 0);
    }
    __device__ __forceinline__ static float get(const Acc &c, int v) { return c.a[v]; }
    // output row of item v in lane group q (f32 result layout)
    __device__ __forceinline__ static int row(int q, int v) { return 4 * q + v; }
};
template <> struct InvMma<double> {
    typedef double v4 __attribute__((ext_vector_type(4)));
    struct Acc { v4 a; };
    __device__ __forceinline__ static void zero(Acc &c) { c.a = v4{0.0, 0.0, 0.0, 0.0}; }
    __device__ __forceinline__ static void mma(double x, double y, Acc &c) {
        c.a = __builtin_amdgcn_mfma_f64_16x16x4f64(x, y, c.a, 0, 0, 0);
    }
    __device__ __forceinline__ static double get(const Acc &c, int v) { return c.a[v]; }
    __device__ __forceinline__ static int row(int q, int v) { return q + 4 * v; }  // f64 layout
};
// complex: four real products (re += xr yr - xi yi, im += xr yi + xi yr)
template <typename C, typename R> struct InvMmaCplx {
    using Re = InvMma<R>;
    struct Acc { typename Re::Acc re, im; };
    __device__ __forceinline__ static void zero(Acc &c) { Re::zero(c.re); Re::zero(c.im); }
    __device__ __forceinline__ static void mma(C x, C y, Acc &c) {
        Re::mma(x.re, y.re, c.re);
        Re::mma(-x.im, y.im, c.re);
        Re::mma(x.re, y.im, c.im);
        Re::mma(x.im, y.re, c.im);
    }
    __device__ __forceinline__ static C get(const Acc &c, int v) { return C{Re::get(c.re, v), Re::get(c.im, v)}; }
    __device__ __forceinline__ static int row(int q, int v) { return Re::row(q, v); }
};
template <> struct InvMma<cplx> : InvMmaCplx<cplx, double> {};
template <> struct InvMma<cplx32> : InvMmaCplx<cplx32, float> {};

// 1/d without a branch (the same values as Elem<T>::recip: a real complex
// divisor gives the exactly rounded real reciprocal); a branch per row of the
// unrolled substitution below split it into divergent blocks whose reads of
// L the compiler then held in registers all at once
__device__ __forceinline__ float recip_nb(float d) { return 1.0f / d; }
__device__ __forceinline__ double recip_nb(double d) { return 1.0 / d; }
__device__ __forceinline__ cplx recip_nb(cplx d) {
    const double den = d.re * d.re + d.im * d.im;
    const bool real = d.im == 0.0;
    return cplx{real ? 1.0 / d.re : d.re / den, real ? 0.0 : -d.im / den};
}
__device__ __forceinline__ cplx32 recip_nb(cplx32 d) {
    const float den = d.re * d.re + d.im * d.im;
    const bool real = d.im == 0.0f;
    return cplx32{real ? 1.0f / d.re : d.re / den, real ? 0.0f : -d.im / den};
}

__device__ __forceinline__ float neg(float x) { return -x; }
__device__ __forceinline__ double neg(double x) { return -x; }
__device__ __forceinline__ cplx neg(cplx x) { return cplx{-x.re, -x.im}; }
__device__ __forceinline__ cplx32 neg(cplx32 x) { return cplx32{-x.re, -x.im}; }

template <typename T, int NB>
__global__ __launch_bounds__(256) void inv_block_kernel(int64_t m, const T *__restrict__ A, int64_t lda,
                                                        T *__restrict__ W, int ldw, int nblk, int nzc) {
    using E = Elem<T>;
    using M = InvMma<T>;
    constexpr int LD = NB + 1;  // LDS column stride
    constexpr bool kCplx = sizeof(T) > sizeof(typename E::Real);
    __shared__ T S[NB * LD];
    // complex: the 16 x 16 inverses are built in LDS (register arrays of
    // complex values made the compiler spill)
    __shared__ T Wsub[kCplx ? NB * 16 : 1];
    const int tid = threadIdx.x;
    const int bid = blockIdx.x;
    const int64_t W2 = (int64_t)ldw * ldw;

    if (bid >= nblk) {
        // zeros in rows [lo, lo + NB) of the parent, columns right of the block
        const int z = bid - nblk;
        const int t = z / nzc, cc = z - (z / nzc) * nzc;
        const int64_t base = (int64_t)t * NB;
        const int64_t tp = base / ldw;
        const int lo = (int)(base - tp * ldw);
        const int bsp = (int)((m - tp * ldw) < ldw ? (m - tp * ldw) : ldw);
        const int rows = (bsp - lo) < NB ? (bsp - lo) : NB;
        const int c0 = lo + NB + 64 * cc;
        const int c1 = (c0 + 64) < bsp ? (c0 + 64) : bsp;
        if (rows <= 0 || c0 >= c1) return;
        T *Wp = W + tp * W2;
        for (int e = tid; e < NB * 64; e += 256) {
            const int i = e % NB, j = e / NB;
            if (i < rows && c0 + j < c1) Wp[(lo + i) + (int64_t)(c0 + j) * ldw] = E::zero();
        }
        return;
    }

    const int64_t base = (int64_t)bid * NB;
    const int bs = (int)((m - base) < NB ? (m - base) : NB);
    const int64_t tp = base / ldw;
    const int lo = (int)(base - tp * ldw);
    T *__restrict__ Wt = W + tp * W2 + (int64_t)lo * (ldw + 1);
    const T *__restrict__ Ad = A + base + base * lda;

    // 1. lower triangle into LDS; every address read lies inside L (indices
    // clamped to the block), so the loads need no condition and all of them
    // are issued before the first LDS write (one memory latency, not one per
    // group of loads)
    {
        constexpr int PER = NB * NB / 256;
        T x[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + 256 * u;
            const int i = e % NB, j = e / NB;
            const int ic = i < bs ? i : bs - 1, jc = j < bs ? j : bs - 1;
            x[u] = Ad[ic + (int64_t)jc * lda];
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + 256 * u;
            const int i = e % NB, j = e / NB;
            const bool in = i < bs && j < bs;
            S[i + j * LD] = E::sel(i >= j && in, x[u], E::sel(i == j, E::one(), E::zero()));
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15;
    const int q = lane >> 4;

    // 2. 16 x 16 diagonal blocks: block d = 4 * wave + q, column j = c16.
    // Row i of column j: (e_j - sum_{k < i} l_ik w_kj) / l_ii; rows above j
    // are zero (set, not computed: a zero l_kk must not turn them into NaN).
    if constexpr (kCplx) {
        const int d = 4 * wave + q;
        if (d < NB / 16) {
            T *Ld = S + d * 16 * (LD + 1);
            T *Wl = Wsub + d * 256 + c16 * 16;  // column c16 of this block's inverse
            for (int i = 0; i < 16; ++i) {
                T acc = E::sel(i == c16, E::one(), E::zero());
#pragma unroll 4
                for (int k = c16; k < i; ++k) acc = E::msub(acc, Ld[i + k * LD], Wl[k]);
                Wl[i] = E::sel(i >= c16, E::mul(acc, recip_nb(Ld[i + i * LD])), E::zero());
            }
            // every lane of the block's group has finished reading L (one
            // wave, in order) before its column is written over L's
            for (int i = 0; i < 16; ++i) Ld[i + c16 * LD] = Wl[i];
        }
    } else {
        const int d = 4 * wave + q;
        if (d < NB / 16) {
            T *Ld = S + d * 16 * (LD + 1);
            T w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                T acc = E::sel(i == c16, E::one(), E::zero());
#pragma unroll
                for (int k = 0; k < i; ++k) acc = E::msub(acc, Ld[i + k * LD], w[k]);
                w[i] = E::sel(i >= c16, E::mul(acc, recip_nb(Ld[i + i * LD])), E::zero());
                // one row at a time: hoisting every row's reads of L would
                // hold 136 elements in registers (spills for complex types)
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) Ld[i + c16 * LD] = w[i];
        }
    }
    __syncthreads();

    // 3. doubling: pairs of b x b blocks at o = 2 b p
#pragma unroll
    for (int b = 16; b < NB; b *= 2) {
        const int nt = b / 16;           // tiles per side
        const int ntile = (NB / (2 * b)) * nt * nt;
        // T = W22 L21 into the upper-right quadrant (W22 lower: k < 16 (ti + 1));
        // tile t of a pair is (t / nt, t % nt), so the waves (t = wave + 4i)
        // share out the row tiles, whose K differs, evenly
        for (int t = wave; t < ntile; t += 4) {
            const int pr = t / (nt * nt), tt = t - pr * nt * nt;
            const int ti = tt / nt, tj = tt - ti * nt;
            const int o = 2 * b * pr;
            const T *Aw = S + (o + b) + (o + b) * LD + ti * 16;
            const T *Bl = S + (o + b) + o * LD + tj * 16 * LD;
            typename M::Acc acc;
            M::zero(acc);
            for (int k0 = 0; k0 < 16 * (ti + 1); k0 += 16)  // 16 k per step: four products
#pragma unroll
                for (int kk = k0; kk < k0 + 16; kk += 4)
                    M::mma(Aw[c16 + (kk + q) * LD], Bl[(kk + q) + c16 * LD], acc);
            T *Dq = S + o + (o + b) * LD + ti * 16 + tj * 16 * LD;
#pragma unroll
            for (int v = 0; v < 4; ++v) Dq[M::row(q, v) + c16 * LD] = M::get(acc, v);
        }
        __syncthreads();
        // X21 = -T W11 over L21 (W11 lower: k >= 16 tj); here the column
        // tiles differ in K, so tile t of a pair is (t % nt, t / nt)
        for (int t = wave; t < ntile; t += 4) {
            const int pr = t / (nt * nt), tt = t - pr * nt * nt;
            const int tj = tt / nt, ti = tt - tj * nt;
            const int o = 2 * b * pr;
            const T *Aq = S + o + (o + b) * LD + ti * 16;
            const T *Bw = S + o + o * LD + tj * 16 * LD;
            typename M::Acc acc;
            M::zero(acc);
            for (int k0 = 16 * tj; k0 < b; k0 += 16)
#pragma unroll
                for (int kk = k0; kk < k0 + 16; kk += 4)
                    M::mma(Aq[c16 + (kk + q) * LD], Bw[(kk + q) + c16 * LD], acc);
            T *Dx = S + (o + b) + o * LD + ti * 16 + tj * 16 * LD;
#pragma unroll
            for (int v = 0; v < 4; ++v) Dx[M::row(q, v) + c16 * LD] = neg(M::get(acc, v));
        }
        __syncthreads();
        // the quadrants used for T are zero in the inverse
        for (int e = tid; e < (NB / (2 * b)) * b * b; e += 256) {
            const int pr = e / (b * b), r = e - pr * b * b;
            const int i = r % b, j = r / b;
            S[(2 * b * pr + i) + (2 * b * pr + b + j) * LD] = E::zero();
        }
        __syncthreads();
    }

    // 4. the block (zeros above its diagonal included) into W
#pragma unroll 8
    for (int e = tid; e < NB * NB; e += 256) {
        const int i = e % NB, j = e / NB;
        if (i < bs && j < bs) Wt[i + (int64_t)j * ldw] = S[i + j * LD];
    }
}

template <typename T, int NB>
hipError_t launch_block(int64_t m, const void *A, int64_t lda, void *W, int ldw, hipStream_t st) {
    const int64_t nblk = (m + NB - 1) / NB;
    if (nblk <= 0) return hipSuccess;
    if (ldw % NB != 0) return hipErrorInvalidValue;
    const int nzc = (ldw - NB) / 64;  // zero tasks per block (columns right of it, 64 each)
    const int64_t grid = nblk * (1 + nzc);
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((inv_block_kernel<T, NB>), dim3((unsigned)grid), dim3(256), 0, st, m,
                       static_cast<const T *>(A), lda, static_cast<T *>(W), ldw, (int)nblk, nzc > 0 ? nzc : 1);
    return hipGetLastError();
}

// Block size of the fused base: 128, 64 for complex fp64 (LDS), never
// more than ib.
int fused_base(int dtype, int ib) {
    const int nb = dtype == C64F ? 64 : 128;
    return ib < nb ? ib : nb;
}

bool use_fused_base() {
    const char *e = std::getenv("TRSM_INV_BASE");
    return !(e && std::strcmp(e, "subst") == 0);
}

hipError_t launch_fused(int dtype, int nbase, int64_t m, const void *A, int64_t lda, void *W, int ldw,
                        hipStream_t st) {
    switch (dtype) {
        case R32F: return nbase == 128 ? launch_block<float, 128>(m, A, lda, W, ldw, st)
                                       : launch_block<float, 64>(m, A, lda, W, ldw, st);
        case R64F: return nbase == 128 ? launch_block<double, 128>(m, A, lda, W, ldw, st)
                                       : launch_block<double, 64>(m, A, lda, W, ldw, st);
        case C32F: return nbase == 128 ? launch_block<cplx32, 128>(m, A, lda, W, ldw, st)
                                       : launch_block<cplx32, 64>(m, A, lda, W, ldw, st);
        case C64F: return launch_block<cplx, 64>(m, A, lda, W, ldw, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t diag_inv_tmp_elems(int ib, int64_t m) {
    if (ib <= kBase || m <= 0) return 0;
    const int64_t nb = (m + ib - 1) / ib;
    return nb * (int64_t)ib * (ib / 2) / 2;  // the largest level, b = ib/2
}

hipError_t diag_inv_launch(int dtype, int ib, int64_t m, const void *A, int64_t lda, void *W,
                           void *tmp, hipStream_t stream) {
    if (ib != 64 && ib != 128 && ib != 256 && ib != 512 && ib != 1024) return hipErrorInvalidValue;
    if (m <= 0) return hipSuccess;
    // the base blocks: the fused NB x NB kernel (TRSM_INV_BASE=subst: the
    // 64 x 64 substitution, for comparison), then doubling from there
    int nbase = kBase;
    hipError_t e;
    if (use_fused_base()) {
        nbase = fused_base(dtype, ib);
        e = launch_fused(dtype, nbase, m, A, lda, W, ib, stream);
    } else {
        e = launch_base(dtype, m, A, lda, W, ib, stream);
    }
    if (e != hipSuccess || ib <= nbase) return e;
    if (tmp == nullptr) return hipErrorInvalidValue;
    const int64_t es = (int64_t)dtype_size(dtype);
    const int64_t nb = (m + ib - 1) / ib;
    const int64_t bsl = m - (nb - 1) * ib;  // rows of the last ib block
    const char *Ab = static_cast<const char *>(A);
    char *Wb = static_cast<char *>(W);
    char *Tb = static_cast<char *>(tmp);
    const Scalar zero{0.0, 0.0}, one{1.0, 0.0}, minus_one{-1.0, 0.0};
    for (int64_t b = nbase; b < ib; b *= 2) {
        // pairs of b x b blocks: pair (zo, zi) starts at row/column
        // o = zo*ib + zi*2b; W11 at (o, o), W22 and L22 at (o+b, o+b),
        // L21 and X21 at (o+b, o); the product W22 L21 goes to tmp
        // (b x b, ld b, pair after pair)
        const int64_t pp = ib / (2 * b);
        const int64_t full_last = bsl / (2 * b);
        const int64_t nfull = (nb - 1) * pp + full_last;
        if (nfull > 0) {
            GemmDesc g1{};  // tmp = W22 * L21
            g1.M = g1.N = g1.K = b;
            g1.A = Wb + b * (1 + ib) * es;
            g1.lda = ib;
            g1.a_lower = 1;
            g1.Bm = Ab + b * es;
            g1.ldb = lda;
            g1.D = Tb;
            g1.ldd = b;
            g1.ldc = b;
            g1.ldd2 = b;
            g1.beta = zero;
            g1.gamma = one;
            g1.batch = nfull;
            g1.binner = pp;
            g1.sAo = (int64_t)ib * ib;
            g1.sAi = 2 * b * (1 + ib);
            g1.sBo = (int64_t)ib * (1 + lda);
            g1.sBi = 2 * b * (1 + lda);
            g1.sDo = pp * b * b;
            g1.sDi = b * b;
            if ((e = gemm_launch(dtype, g1, stream)) != hipSuccess) return e;
            GemmDesc g2{};  // X21 = -tmp * W11
            g2.M = g2.N = g2.K = b;
            g2.A = Tb;
            g2.lda = b;
            g2.Bm = Wb;
            g2.ldb = ib;
            g2.D = Wb + b * es;
            g2.ldd = ib;
            g2.ldc = ib;
            g2.ldd2 = ib;
            g2.beta = zero;
            g2.gamma = minus_one;
            g2.b_lower = 1;
            g2.batch = nfull;
            g2.binner = pp;
            g2.sAo = pp * b * b;
            g2.sAi = b * b;
            g2.sBo = (int64_t)ib * ib;
            g2.sBi = 2 * b * (1 + ib);
            g2.sDo = (int64_t)ib * ib;
            g2.sDi = 2 * b * (1 + ib);
            if ((e = gemm_launch(dtype, g2, stream)) != hipSuccess) return e;
        }
        // a last pair whose second block is cut short by the end of L
        const int64_t o = 2 * b * full_last;
        const int64_t r = bsl - o - b;  // rows of its second block, < b
        if (r > 0) {
            const char *Wt = Wb + (nb - 1) * ib * ib * es;
            const char *At = Ab + (nb - 1) * ib * (1 + lda) * es;
            GemmDesc g1{};
            g1.M = g1.K = r;
            g1.N = b;
            g1.A = Wt + (o + b) * (1 + ib) * es;
            g1.lda = ib;
            g1.a_lower = 1;
            g1.Bm = At + ((o + b) + o * lda) * es;
            g1.ldb = lda;
            g1.D = Tb;
            g1.ldd = b;
            g1.ldc = b;
            g1.ldd2 = b;
            g1.beta = zero;
            g1.gamma = one;
            if ((e = gemm_launch(dtype, g1, stream)) != hipSuccess) return e;
            GemmDesc g2{};
            g2.M = r;
            g2.N = g2.K = b;
            g2.A = Tb;
            g2.lda = b;
            g2.Bm = Wt + o * (1 + ib) * es;
            g2.ldb = ib;
            g2.D = const_cast<char *>(Wt) + ((o + b) + o * ib) * es;
            g2.ldd = ib;
            g2.ldc = ib;
            g2.ldd2 = ib;
            g2.beta = zero;
            g2.gamma = minus_one;
            g2.b_lower = 1;
            if ((e = gemm_launch(dtype, g2, stream)) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace trsm
