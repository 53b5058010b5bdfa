// Kernel (a) on the matrix cores: the direct solve of L X = alpha B for
// m <= 64 in fp64 and complex fp64, one workgroup per (problem, group of 64
// right-hand-side columns).
//
// HSMA-TRSM ("Hierarchical Shared Memory-Aware Optimization for TRSM on GPU
// Platforms") keeps a small problem on chip and solves it in one thread
// block (section 4.2.1); its large-regime machinery (section 4.3) inverts
// the diagonal blocks and turns the rest into matrix products.  On gfx950
// the whole small problem fits one workgroup's LDS and registers, and the
// fp64 matrix cores run at the same rate as the fp64 vector units while
// needing no per-product LDS broadcast, so the small solve is done as the
// blocked algorithm at 16 x 16 granularity inside one workgroup:
//
//   * the lower 16 x 16 blocks of L (ten of them, 40 KB for complex) are
//     staged in LDS; rows past m become identity rows; every element of A
//     and B moves by a raw buffer operation with no branch around it, so all
//     of a thread's loads are in flight at once and its stores go out
//     back to back (guarded loads made the compiler wait for each one);
//   * one wave inverts the four diagonal blocks in place (lane group g takes
//     block g) by substitution against the columns of the identity (section
//     4.3.1's column-streamed inversion at 16 x 16 scale);
//   * wave w then owns right-hand-side columns 16w .. 16w+15 of the group,
//     all 64 rows of them as v_mfma_f64_16x16x4f64 accumulators, and for
//     p = 0..3 computes X_p = W_p B_p and B_q -= L_qp X_p (q > p) without
//     further synchronisation: the f64 MFMA result layout (row g + 4v in
//     item v of lane group g) is exactly the layout of its B operand, so a
//     solved panel feeds the next products straight from the accumulators;
//   * complex fp64 uses the real 2x2 embedding (4 real products per complex
//     product), expanded from the complex LDS blocks when the A fragments
//     are read.
// Four waves per workgroup and three (complex) or four (fp64) workgroups
// per CU, so one workgroup's loads overlap the others' products.
#include "buffer_ops.h"
#include "scalar_ops.h"

namespace trsm {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef double d2v __attribute__((ext_vector_type(2)));

constexpr int kPanels = 4;  // 16-row panels of the 64 rows
__host__ __device__ constexpr int blk(int q, int p) { return q * (q + 1) / 2 + p; }

// A fragment for k-step s of the product (output tile a) x (input tile t)
// with the 16 x 16 block Lb (stored [k][i]); `neg` flips the sign.
// fp64: MFMA row r stands for block row 4(r % 4) + r / 4, so that item v
// of lane group g holds block row 4g + v; the k row of a B operand item
// (4s + g) is block row 4g + s.
__device__ __forceinline__ double afrag(const double (*Lb)[16], int a, int t, int s, int c, int g,
                                        double sgn) {
    (void)a;
    (void)t;
    return sgn * Lb[4 * g + s][4 * (c & 3) + (c >> 2)];
}
// complex: real row r of an 8-complex-row tile stands for complex row
// (r % 4) + 4 (r / 8), part (r / 4) % 2; item v of lane group g then holds
// complex rows g (v = 0, 1: re, im) and g + 4 (v = 2, 3) of the tile.
__device__ __forceinline__ double afrag(const cplx (*Lb)[16], int a, int t, int s, int c, int g,
                                        double sgn) {
    const int i = (c & 3) + 4 * (c >> 3) + 8 * a;
    const int ri = (c >> 2) & 1;
    const int k = g + 4 * (s >> 1) + 8 * t;
    const int ki = s & 1;
    const cplx z = Lb[k][i];
    const double v = (ri == ki) ? z.re : (ri ? z.im : -z.im);
    return sgn * v;
}

// One element of A through a raw buffer load; `ok == false` reads nothing
// (an offset past the range returns zero without a memory access).
template <typename T>
__device__ __forceinline__ T ld_elem(__amdgpu_buffer_rsrc_t r, int64_t idx, bool ok) {
    const uint32_t off = ok ? (uint32_t)(idx * (int64_t)sizeof(T)) : 0xfffffff0u;
    if constexpr (sizeof(T) == 16) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    } else {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
}

// One element of B written through a raw buffer store; `ok == false` writes
// nothing (a store past the range is dropped).
template <typename T>
__device__ __forceinline__ void st_elem(__amdgpu_buffer_rsrc_t r, int64_t idx, bool ok, T v) {
    const uint32_t off = ok ? (uint32_t)(idx * (int64_t)sizeof(T)) : 0xfffffff0u;
    if constexpr (sizeof(T) == 16) {
        typedef unsigned u4t __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4t, v), r, off, 0, 0);
    } else {
        typedef unsigned u2t __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2t, v), r, off, 0, 0);
    }
}

// BUF: one problem's A and B each span less than 2^31 bytes, so they are
// read and written with branch-free buffer operations, all in flight
// together (a guarded access per element makes the compiler wait for each
// one before the next).
template <typename T, bool BUF>
__global__ __launch_bounds__(256) void small_mfma_kernel(int m, int64_t n, int64_t ncg,
                                                         Scalar alpha_s, const T *__restrict__ A,
                                                         int64_t lda, int64_t strideA,
                                                         T *__restrict__ B, int64_t ldb,
                                                         int64_t strideB) {
    using E = Elem<T>;
    constexpr bool CPLX = sizeof(T) == 16;
    constexpr int TILES = CPLX ? 2 : 1;  // 16-real-row MFMA tiles per 16-row panel
    __shared__ __attribute__((aligned(16))) T Lb[10][16][16];  // block (q,p): [k][i]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int64_t prob = blockIdx.x / ncg;
    const int64_t cgi = blockIdx.x - prob * ncg;
    const T *__restrict__ Ap = A + prob * strideA;
    T *__restrict__ Bp = B + prob * strideB;
    const int np = (m + 15) >> 4;  // panels that hold rows < m

    // ---- 1. this wave's 16 columns, all rows, into accumulators ----------
    // B does not depend on L, so its loads are in flight while L is staged
    // and inverted (measured faster than loading B after the inversion,
    // although the longer register life leaves three waves per SIMD for
    // complex instead of four).  With buffer loads they are issued right
    // after L's: loads complete in order, so waiting for L then leaves B in
    // flight, and panel p of the solve below waits only for its own rows.
    const int64_t col = cgi * 64 + w * 16 + c;
    const bool colok = col < n;
    T *__restrict__ Bc = Bp + col * ldb;
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(Bp, BUF ? ((n - 1) * ldb + m) * (int64_t)sizeof(T) : 0);
    d4 acc[kPanels][TILES];
    auto load_b = [&]() {
#pragma unroll
    for (int p = 0; p < kPanels; ++p) {
#pragma unroll
        for (int a = 0; a < TILES; ++a) {
            if constexpr (BUF && CPLX) {
                const int r0 = 16 * p + 8 * a + g;
                const cplx z0 = ld_elem<cplx>(rsb, r0 + col * ldb, colok && r0 < m);
                const cplx z1 = ld_elem<cplx>(rsb, r0 + 4 + col * ldb, colok && r0 + 4 < m);
                acc[p][a] = d4{z0.re, z0.im, z1.re, z1.im};
            } else if constexpr (BUF) {
                const int r0 = 16 * p + 4 * g;
                double v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = ld_elem<double>(rsb, r0 + e + col * ldb, colok && r0 + e < m);
                acc[p][a] = d4{v[0], v[1], v[2], v[3]};
            } else if constexpr (CPLX) {
                const int r0 = 16 * p + 8 * a + g;  // complex rows r0 and r0 + 4
                cplx z0{0.0, 0.0}, z1{0.0, 0.0};
                if (colok && r0 < m) z0 = Bc[r0];
                if (colok && r0 + 4 < m) z1 = Bc[r0 + 4];
                acc[p][a] = d4{z0.re, z0.im, z1.re, z1.im};
            } else {
                const int r0 = 16 * p + 4 * g;  // rows r0 .. r0 + 3
                double v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (colok && r0 + e < m) ? Bc[r0 + e] : 0.0;
                acc[p][a] = d4{v[0], v[1], v[2], v[3]};
            }
        }
    }

    };
    if constexpr (!BUF) load_b();

    // ---- 2. lower blocks of L into LDS (rows >= m: identity) ---------------
    {
        const int i = tid & 15, k = tid >> 4;
        if constexpr (BUF) {
            // all ten loads first, then the masks and the LDS writes
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(Ap, ((int64_t)(m - 1) * lda + m) * (int64_t)sizeof(T));
            T v[kPanels * (kPanels + 1) / 2];
#pragma unroll
            for (int q = 0; q < kPanels; ++q)
#pragma unroll
                for (int p = 0; p <= q; ++p) {
                    const int gi = 16 * q + i, gk = 16 * p + k;
                    v[blk(q, p)] = ld_elem<T>(rs, gi + (int64_t)gk * lda, gi < m && gk < m && gi >= gk);
                }
            load_b();  // B's loads behind L's (see phase 1)
#pragma unroll
            for (int q = 0; q < kPanels; ++q)
#pragma unroll
                for (int p = 0; p <= q; ++p) {
                    const int gi = 16 * q + i, gk = 16 * p + k;
                    // out-of-range reads came back zero; rows past m get a 1
                    // on the diagonal
                    Lb[blk(q, p)][k][i] = E::sel(gi == gk && gi >= m, E::one(), v[blk(q, p)]);
                }
        } else {
#pragma unroll
            for (int q = 0; q < kPanels; ++q) {
#pragma unroll
                for (int p = 0; p <= q; ++p) {
                    const int gi = 16 * q + i, gk = 16 * p + k;
                    T v = E::zero();
                    if (gi < m && gk < m) {
                        if (gi >= gk) v = Ap[gi + (int64_t)gk * lda];
                    } else if (gi == gk) {
                        v = E::one();
                    }
                    Lb[blk(q, p)][k][i] = v;
                }
            }
        }
    }
    __syncthreads();

    // ---- 3. wave 0 inverts the diagonal blocks in place --------------------
    // Lane group g takes block g, lane c of it column c of the inverse.  The
    // pivots' reciprocals are computed first (one per lane) and stored over
    // the diagonal, so the substitution itself only multiplies.
    if (w == 0 && g < np) {
        T(*D)[16] = Lb[blk(g, g)];
        D[c][c] = E::recip(D[c][c]);
        T x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (i == c) ? E::one() : E::zero();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            x[k] = E::mul(x[k], D[k][k]);
#pragma unroll
            for (int i = k + 1; i < 16; ++i) x[i] = E::msub(x[i], D[k][i], x[k]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) D[c][i] = x[i];
    }
    __syncthreads();

    // ---- 4. B_p -= sum_{q<p} L_pq X_q, then X_p = W_p B_p ------------------
    // Panel p takes the updates of the panels above it just before its own
    // product (the same updates in the same order as updating every panel
    // below as soon as a panel is solved), so the products of panel p need
    // only B_p and the solved panels: the rows of later panels may still be
    // arriving.
    const T alpha = E::from(alpha_s);
#pragma unroll
    for (int p = 0; p < kPanels; ++p) {
        if (p < np) {  // uniform
#pragma unroll
        for (int q = 0; q < p; ++q)
#pragma unroll
            for (int a = 0; a < TILES; ++a)
#pragma unroll
                for (int t = 0; t < TILES; ++t)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc[p][a] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                            afrag(Lb[blk(p, q)], a, t, s, c, g, -1.0), acc[q][t][s], acc[p][a], 0, 0, 0);
        d4 x[TILES];
#pragma unroll
        for (int a = 0; a < TILES; ++a) {
            x[a] = d4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int t = 0; t <= a; ++t)  // W_p is lower triangular: tile (0, 1) is zero
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    x[a] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                        afrag(Lb[blk(p, p)], a, t, s, c, g, 1.0), acc[p][t][s], x[a], 0, 0, 0);
        }
        // X_p replaces B_p in the accumulators; the stores wait until the end,
        // so no panel's products wait for another panel's stores to drain
#pragma unroll
        for (int a = 0; a < TILES; ++a) acc[p][a] = x[a];
        }
    }

    // ---- 5. B <- alpha X ---------------------------------------------------
#pragma unroll
    for (int p = 0; p < kPanels; ++p) {
#pragma unroll
        for (int a = 0; a < TILES; ++a) {
            if constexpr (BUF && CPLX) {
                const int r0 = 16 * p + 8 * a + g;
                st_elem<cplx>(rsb, r0 + col * ldb, colok && r0 < m, E::mul(alpha, cplx{acc[p][a][0], acc[p][a][1]}));
                st_elem<cplx>(rsb, r0 + 4 + col * ldb, colok && r0 + 4 < m,
                              E::mul(alpha, cplx{acc[p][a][2], acc[p][a][3]}));
            } else if constexpr (BUF) {
                const int r0 = 16 * p + 4 * g;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    st_elem<double>(rsb, r0 + e + col * ldb, colok && r0 + e < m, alpha * acc[p][a][e]);
            } else if constexpr (CPLX) {
                const int r0 = 16 * p + 8 * a + g;
                if (colok && r0 < m) Bc[r0] = E::mul(alpha, cplx{acc[p][a][0], acc[p][a][1]});
                if (colok && r0 + 4 < m) Bc[r0 + 4] = E::mul(alpha, cplx{acc[p][a][2], acc[p][a][3]});
            } else {
                const int r0 = 16 * p + 4 * g;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (colok && r0 + e < m) Bc[r0 + e] = alpha * acc[p][a][e];
            }
        }
    }
}

}  // namespace

hipError_t small_mfma_launch(int dtype, int m, int64_t n, Scalar alpha, const void *A,
                             int64_t lda, int64_t strideA, void *B, int64_t ldb, int64_t strideB,
                             int64_t batch, hipStream_t stream) {
    if (m < 1 || m > 64) return hipErrorInvalidValue;
    const int64_t ncg = (n + 63) / 64;
    const int64_t nblk = ncg * batch;
    if (nblk <= 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // one problem's A and B in 32-bit buffer offsets (with room for the
    // past-the-end offset of skipped elements)
    const int64_t es = dtype == C64F ? 16 : 8;
    const bool buf = ((int64_t)(m - 1) * lda + m) * es < 0x7fffffffLL &&
                     (n - 1) <= (0x7fffffffLL / es - m) / (ldb > 0 ? ldb : 1);
    const dim3 grid((unsigned)nblk);
    switch (dtype) {
        case R64F:
            if (buf)
                hipLaunchKernelGGL((small_mfma_kernel<double, true>), grid, dim3(256), 0, stream, m, n, ncg, alpha,
                                   static_cast<const double *>(A), lda, strideA, static_cast<double *>(B), ldb, strideB);
            else
                hipLaunchKernelGGL((small_mfma_kernel<double, false>), grid, dim3(256), 0, stream, m, n, ncg, alpha,
                                   static_cast<const double *>(A), lda, strideA, static_cast<double *>(B), ldb, strideB);
            break;
        case C64F:
            if (buf)
                hipLaunchKernelGGL((small_mfma_kernel<cplx, true>), grid, dim3(256), 0, stream, m, n, ncg, alpha,
                                   static_cast<const cplx *>(A), lda, strideA, static_cast<cplx *>(B), ldb, strideB);
            else
                hipLaunchKernelGGL((small_mfma_kernel<cplx, false>), grid, dim3(256), 0, stream, m, n, ncg, alpha,
                                   static_cast<const cplx *>(A), lda, strideA, static_cast<cplx *>(B), ldb, strideB);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace trsm
