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
//   * wave w inverts diagonal block w in place by substitution against the
//     columns of the identity (section 4.3.1's column-streamed inversion at
//     16 x 16 scale), each column spread over a lane quad;
//   * wave w then owns right-hand-side columns 16w .. 16w+15 of the group,
//     all 64 rows of them as v_mfma_f64_16x16x4f64 accumulators, and for
//     p = 0..3 computes X_p = W_p B_p and B_q -= L_qp X_p (q > p) without
//     further synchronisation: the f64 MFMA result layout (row g + 4v in
//     item v of lane group g) is exactly the layout of its B operand, so a
//     solved panel feeds the next products straight from the accumulators;
//   * complex fp64 uses the real 2x2 embedding (4 real products per complex
//     product), expanded from the complex LDS blocks when the A fragments
//     are read.
// Four waves per workgroup and three (complex, by registers) or six (fp64)
// workgroups per CU, so one workgroup's loads overlap the others' products.
#include <cstdlib>
#include <map>
#include <mutex>

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

// v from lane r of this lane's quad (DPP quad permute; r must fold to a
// constant)
__device__ __forceinline__ int quad_bcast_w(int v, int r) {
    switch (r) {
    case 0: return __builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false);
    case 1: return __builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false);
    default: return __builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false);
    }
}
template <typename T> __device__ __forceinline__ T quad_bcast(T v, int r) {
    struct Words { int w[sizeof(T) / 4]; };
    Words a = __builtin_bit_cast(Words, v);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) a.w[i] = quad_bcast_w(a.w[i], r);
    return __builtin_bit_cast(T, a);
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
    // and inverted (measured faster than loading B after the inversion).
    // With buffer loads they are issued right
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

    // ---- 3. the diagonal blocks are inverted in place, block w by wave w ---
    // Lane 4c + r takes column c of the inverse, rows r, r + 4, r + 8 and
    // r + 12, so each column is spread over one lane quad.  The pivots'
    // reciprocals are stored over the diagonal first.  At step k the lane
    // that holds row k scales it by the reciprocal, a quad permute hands the
    // scaled value to the quad's other lanes, and each lane subtracts its
    // multiples of it from its rows below k.
    if (w < np) {
        const int ic = lane >> 2, ir = lane & 3;
        T(*D)[16] = Lb[blk(w, w)];
        if (ir == 0) D[ic][ic] = E::recip(D[ic][ic]);
        T x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (4 * j + ir == ic) ? E::one() : E::zero();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int jk = k >> 2, rk = k & 3;
            const T xk = quad_bcast(E::mul(x[jk], D[k][k]), rk);
            const T u = E::msub(x[jk], D[k][4 * jk + ir], xk);
            x[jk] = E::sel(ir > rk, u, E::sel(ir == rk, xk, x[jk]));
#pragma unroll
            for (int j = jk + 1; j < 4; ++j) x[j] = E::msub(x[j], D[k][4 * j + ir], xk);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) D[ic][4 * j + ir] = x[j];
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

// ---- producer/consumer form for large batches of complex fp64 problems ----
//
// HSMA-TRSM, section 4.2.2 and Figure 5: for the complex fp64 case, whose
// operands strain on-chip memory, the pages split each thread block into a
// group that moves data and a group that computes, and pipeline the two.
// On gfx950 the split is by wavefront inside one persistent workgroup per
// CU that loops over (problem, 64-column group) tasks:
//   * wave 4, the producer, streams the next task's ten lower 16 x 16 blocks
//     of L and its 64 x 64 block of B from HBM straight into LDS with
//     direct-to-LDS buffer loads (no registers in between; an out-of-range
//     lane writes zeros, which gives the zero rows past m and columns past
//     n), then inverts the next task's four diagonal blocks in place -- the
//     inversion leaves the compute waves' critical path;
//   * waves 0-3, the consumers, copy the current task's B from LDS into
//     their MFMA accumulators, solve as small_mfma_kernel does (16 columns
//     each, blocked substitution with the inverted diagonal blocks), and
//     write X from registers;
//   * L is double-buffered (2 x 40 KB), B single-buffered (64 KB: the
//     consumers hold it in registers after the first moments of a task, so
//     the producer refills it while they compute); each staged column of B
//     has 16 bytes of padding so the consumers' column-strided LDS reads
//     spread over the banks.  148 KB of LDS: one workgroup per CU.
// Two barriers per task, taken by all five waves the same number of times:
//   A(t): L(t) inverted and B(t) staged (the producer has waited for its
//         loads and written its inversion);
//   B(t): the consumers have copied B(t) into registers, so the B buffer is
//         free for task t+1.
constexpr int kPcColPitch = 64 * 16 + 16;  // bytes per staged column of B

typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(320) void small_pc_kernel(int m, int64_t n, int64_t ncg, int64_t ntasks,
                                                       Scalar alpha_s, const cplx *__restrict__ A,
                                                       int64_t lda, int64_t strideA,
                                                       cplx *__restrict__ B, int64_t ldb,
                                                       int64_t strideB) {
    using E = Elem<cplx>;
    constexpr int TILES = 2;
    __shared__ __attribute__((aligned(16))) cplx Ls[2][10][16][16];  // block (q,p): [k][i]
    __shared__ __attribute__((aligned(16))) unsigned char Bs[64 * kPcColPitch];

    const int tid = threadIdx.x;
    const int w = tid >> 6;  // 0..3 consumers, 4 producer
    const int np = (m + 15) >> 4;
    // Lane indices, laundered through an empty asm at each use site: values
    // derived from them (fragment addresses, the identity column) are cheap
    // to recompute, and hoisted out of the task loop they would stay live
    // across it and push the kernel past 256 VGPRs.
    auto lane_id = [&]() {
        int l = tid & 63;
        asm volatile("" : "+v"(l));
        return l;
    };
    const cplx alpha = E::from(alpha_s);
    const int64_t a_ext = ((int64_t)(m - 1) * lda + m) * 16;
    const int64_t b_ext = ((n - 1) * ldb + m) * 16;

    // producer: task t's L into buffer buf, and its B
    auto issue_loads = [&](int64_t t, int buf) {
        const int lane = lane_id();
        const int64_t prob = t / ncg;
        const int64_t cg = t - prob * ncg;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + prob * strideA, a_ext);
        const int i = lane & 15, kq = lane >> 4;
        // rolled loops: one offset register, not one per load
#pragma nounroll
        for (int q = 0; q < np; ++q) {  // blocks wholly past m are never read
#pragma nounroll
            for (int p = 0; p <= q; ++p)
#pragma nounroll
                for (int kc = 0; kc < 4; ++kc) {
                    const int gi = 16 * q + i, gk = 16 * p + 4 * kc + kq;
                    const bool ok = gi < m && gk < m && gi >= gk;
                    const uint32_t off = ok ? (uint32_t)((gi + (int64_t)gk * lda) * 16) : 0xfffffff0u;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)&Ls[buf][blk(q, p)][4 * kc][0], 16,
                                                             off, 0, 0, 0);
                }
        }
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + prob * strideB, b_ext);
        const int64_t cols = n - cg * 64 < 64 ? n - cg * 64 : 64;
#pragma nounroll
        for (int j = 0; j < cols; ++j) {
            const int64_t col = cg * 64 + j;
            const uint32_t off = lane < m ? (uint32_t)((lane + col * ldb) * 16) : 0xfffffff0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)&Bs[j * kPcColPitch], 16, off, 0, 0, 0);
        }
    };
    // producer: invert the diagonal blocks of buffer buf in place, lane
    // group g taking block g, lane c column c of its inverse (section 4.3.1's
    // substitution against identity columns); a row past m is an identity
    // row (its loaded pivot is zero)
    auto invert = [&](int buf) {
        const int lane = lane_id();
        const int c = lane & 15, g = lane >> 4;
        if (g >= np) return;
        cplx(*D)[16] = Ls[buf][blk(g, g)];
        D[c][c] = (16 * g + c < m) ? E::recip(D[c][c]) : E::one();
        cplx x[16];
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
    };
    // vmcnt(0): the direct-to-LDS loads have written LDS
    constexpr int kWaitVm0 = 0x0F70;

    int64_t t = blockIdx.x;
    int buf = 0;
    if (w == 4 && t < ntasks) {
        issue_loads(t, 0);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        invert(0);
    }
    __syncthreads();  // A(first task)
    for (; t < ntasks; t += gridDim.x, buf ^= 1) {
        const int64_t tn = t + gridDim.x;
        d4 acc[kPanels][TILES];
        const int lane = lane_id();
        const int c = lane & 15, g = lane >> 4;
        const int col_l = w * 16 + c;  // column of the task's 64 this lane solves
        if (w < 4) {
#pragma unroll
            for (int p = 0; p < kPanels; ++p)
#pragma unroll
                for (int a = 0; a < TILES; ++a) {
                    const int r0 = 16 * p + 8 * a + g;
                    const cplx z0 = *reinterpret_cast<const cplx *>(&Bs[col_l * kPcColPitch + 16 * r0]);
                    const cplx z1 = *reinterpret_cast<const cplx *>(&Bs[col_l * kPcColPitch + 16 * (r0 + 4)]);
                    acc[p][a] = d4{z0.re, z0.im, z1.re, z1.im};
                }
        }
        __syncthreads();  // B(t): the B buffer is free
        if (w == 4) {
            if (tn < ntasks) {
                issue_loads(tn, buf ^ 1);
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
                invert(buf ^ 1);
            }
        } else {
            const cplx(*Lc)[16][16] = Ls[buf];
#pragma unroll
            for (int p = 0; p < kPanels; ++p) {
                if (p < np) {  // uniform
#pragma unroll
                    for (int q = 0; q < p; ++q)
#pragma unroll
                        for (int a = 0; a < TILES; ++a)
#pragma unroll
                            for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
                                for (int s = 0; s < 4; ++s)
                                    acc[p][a] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                                        afrag(Lc[blk(p, q)], a, tt, s, c, g, -1.0), acc[q][tt][s], acc[p][a], 0, 0, 0);
                    d4 x[TILES];
#pragma unroll
                    for (int a = 0; a < TILES; ++a) {
                        x[a] = d4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
                        for (int tt = 0; tt <= a; ++tt)
#pragma unroll
                            for (int s = 0; s < 4; ++s)
                                x[a] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                                    afrag(Lc[blk(p, p)], a, tt, s, c, g, 1.0), acc[p][tt][s], x[a], 0, 0, 0);
                    }
#pragma unroll
                    for (int a = 0; a < TILES; ++a) acc[p][a] = x[a];
                }
            }
            const int64_t prob = t / ncg;
            const int64_t col = (t - prob * ncg) * 64 + col_l;
            const bool colok = col < n;
            const __amdgpu_buffer_rsrc_t rsb = make_rsrc(B + prob * strideB, b_ext);
#pragma unroll
            for (int p = 0; p < kPanels; ++p)
#pragma unroll
                for (int a = 0; a < TILES; ++a) {
                    const int r0 = 16 * p + 8 * a + g;
                    st_elem<cplx>(rsb, r0 + col * ldb, colok && r0 < m, E::mul(alpha, cplx{acc[p][a][0], acc[p][a][1]}));
                    st_elem<cplx>(rsb, r0 + 4 + col * ldb, colok && r0 + 4 < m,
                                  E::mul(alpha, cplx{acc[p][a][2], acc[p][a][3]}));
                }
        }
        __syncthreads();  // A(t + gridDim.x)
    }
}

int device_cus() {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = cus;
    return cus;
}

// Producer/consumer form for complex fp64: opt-in (TRSM_SMALL_PC=1), for
// tuning and tests.  Measured on MI355X for a batch of 8192 complex 64 x 64
// problems it ran 466 us against 280 us for small_mfma_kernel: with 148 KB
// of LDS one workgroup fits a CU, so one producer wave per CU keeps too few
// loads in flight (its side alone, with the consumers' products skipped,
// took 342 us) and one MFMA wave per SIMD leaves the products' LDS and
// dependency latencies exposed (the consumers' side alone, 359 us); three
// resident workgroup-per-task workgroups per CU hide both.
bool use_small_pc(int64_t ntasks, int cus) {
    (void)ntasks;
    (void)cus;
    const char *e = std::getenv("TRSM_SMALL_PC");
    return e && e[0] == '1';
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
            if (buf) {
                const int cus = device_cus();
                if (cus > 0 && use_small_pc(nblk, cus)) {
                    const int64_t nwg = nblk < cus ? nblk : cus;
                    hipLaunchKernelGGL(small_pc_kernel, dim3((unsigned)nwg), dim3(320), 0, stream, m, n, ncg, nblk,
                                       alpha, static_cast<const cplx *>(A), lda, strideA, static_cast<cplx *>(B),
                                       ldb, strideB);
                    break;
                }
                hipLaunchKernelGGL((small_mfma_kernel<cplx, true>), grid, dim3(256), 0, stream, m, n, ncg, alpha,
                                   static_cast<const cplx *>(A), lda, strideA, static_cast<cplx *>(B), ldb, strideB);
            }
            else
                hipLaunchKernelGGL((small_mfma_kernel<cplx, false>), grid, dim3(256), 0, stream, m, n, ncg, alpha,
                                   static_cast<const cplx *>(A), lda, strideA, static_cast<cplx *>(B), ldb, strideB);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace trsm
