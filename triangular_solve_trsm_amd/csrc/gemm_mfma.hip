// Kernels (b2, b3): the GEMMs of phase 2 of the blocked algorithm on the
// CDNA4 matrix cores.
//
// HSMA-TRSM ("Hierarchical Shared Memory-Aware Optimization for TRSM on GPU
// Platforms"), section 4.3 "Phase 2": each block row r is solved with the
// precomputed inverse, X_r = D_r^{-1} B_r (a GEMM), and the blocks below are
// updated by a GEMM with the off-diagonal panel of L.  Both are instances of
//
//     D = beta * C + gamma * (A * Bm)        (column-major, ragged edges)
//
// with two extras: rows [0, split) of the result can be routed to a second
// destination (the update writes the next block row into the panel buffer
// that the next solve reads, so no copy is needed), and a lower-triangular A
// skips the K-tiles right of each row tile's diagonal (the solve GEMM).
//
// gfx950 mapping:
//   * 256 threads = 2 x 2 wavefronts, macro tile MT x NT (real rows x cols),
//     each wave 64 x 64 built from 4 x 4 tiles of v_mfma_f64_16x16x4f64 (fp64,
//     complex) or v_mfma_f32_16x16x4f32 (fp32, true fp32 products);
//   * operands are staged in LDS, double-buffered: the global loads of K-tile
//     t+1 are in flight while the MFMAs of tile t run, one barrier per tile;
//   * complex fp64 uses the real 2x2 embedding: a complex M x K by K x N
//     product is a real (2M x 2K) by (2K x N) product where each complex
//     a = ar + i ai of A becomes [[ar, -ai], [ai, ar]]; the interleaved
//     storage of Bm is already its real (2K x N) view, the A fragment is
//     expanded on the fly from the complex tile in LDS, and the real rows are
//     ordered so that each lane ends up holding whole complex results.  This
//     is exactly the 4 real products per complex product (no 3M trick);
//   * tiles are mapped so that each XCD (8 per chip, each with its own L2)
//     works on a band of 8 column tiles at a time, and the workgroups of one
//     XCD cover roughly 8 x 8 tiles, sharing the A and Bm panels in its L2.
#include <type_traits>

#include "scalar_ops.h"

namespace trsm {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef double d2v __attribute__((ext_vector_type(2)));

template <typename T> struct GemmTraits;
template <> struct GemmTraits<float> {
    using R = float;
    using Acc = f4;
    using Vec = f4;  // 16-byte global load unit
    static constexpr int kVec = 4;
    static constexpr bool kCplx = false;
    __device__ __forceinline__ static Acc mfma(R a, R b, Acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // Row of the 16x16 result held by item v of a lane in group q = lane/16.
    __device__ __forceinline__ static int out_row(int q, int v) { return 4 * q + v; }
};
template <> struct GemmTraits<double> {
    using R = double;
    using Acc = d4;
    using Vec = d2v;
    static constexpr int kVec = 2;
    static constexpr bool kCplx = false;
    __device__ __forceinline__ static Acc mfma(R a, R b, Acc c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    // The f64 variant interleaves the other way (checked on gfx950).
    __device__ __forceinline__ static int out_row(int q, int v) { return q + 4 * v; }
};
template <> struct GemmTraits<cplx> {
    using R = double;
    using Acc = d4;
    using Vec = d2v;
    static constexpr int kVec = 2;
    static constexpr bool kCplx = true;
    __device__ __forceinline__ static Acc mfma(R a, R b, Acc c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static int out_row(int q, int v) { return q + 4 * v; }
};

template <typename T>
struct GemmParams {
    int64_t M, N, K;  // in elements of T (complex counts for cplx)
    const T *A;
    int64_t lda;
    const T *Bm;
    int64_t ldb;
    const T *C;
    int64_t ldc;
    T *D;
    int64_t ldd;
    T *D2;
    int64_t ldd2;
    int64_t split;
    Scalar beta, gamma;
    int has_c;
    int a_vec;  // 16-byte vector loads of A columns are aligned
    int b_vec;  // same for Bm
    int tilesM, tilesN;
};

// Workgroup -> tile: consecutive workgroups go round-robin to the 8 XCDs, so
// workgroup w runs on XCD w % 8.  Enumerate tiles in bands of 8 column tiles
// (row tile slow, column tile fast inside a band) and give each XCD a
// contiguous run of that order.
__device__ __forceinline__ void map_tile(int w, int tilesM, int tilesN, int &tm, int &tn) {
    const int ntiles = tilesM * tilesN;
    const int x = w & 7;
    const int s = w >> 3;
    const int per = ntiles >> 3;
    const int rem = ntiles & 7;
    const int q = x * per + (x < rem ? x : rem) + s;
    const int band = q / (tilesM * 8);
    const int r = q - band * tilesM * 8;
    const int wb = (tilesN - band * 8) < 8 ? (tilesN - band * 8) : 8;
    tm = r / wb;
    tn = band * 8 + (r - (r / wb) * wb);
}

// TRI: A is lower triangular (the solve GEMM); a separate instantiation so
// that the solve and the update appear as distinct kernels in traces.
template <typename T, int MT, int NT, int KT, bool TRI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams<T> p) {
    using Tr = GemmTraits<T>;
    using R = typename Tr::R;
    using Acc = typename Tr::Acc;
    using Vec = typename Tr::Vec;
    constexpr bool CPLX = Tr::kCplx;
    constexpr int VEC = Tr::kVec;
    constexpr int WM = MT / 2, WN = NT / 2;  // per-wave tile
    constexpr int FM = WM / 16, FN = WN / 16;
    // LDS: A as [k][row] (rows contiguous), Bm as [k][col] (cols contiguous).
    constexpr int PADA = CPLX ? 1 : VEC;  // keeps 16-byte alignment of A rows
    constexpr int PADB = 1;
    constexpr int AROWS = CPLX ? MT / 2 : MT;  // complex rows for cplx
    constexpr int AK = CPLX ? KT / 2 : KT;
    using AS = typename std::conditional<CPLX, cplx, R>::type;
    __shared__ AS As[2][AK][AROWS + PADA];
    __shared__ R Bs[2][KT][NT + PADB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    int tm, tn;
    if (blockIdx.x >= (unsigned)(p.tilesM * p.tilesN)) return;
    map_tile(blockIdx.x, p.tilesM, p.tilesN, tm, tn);

    // Real-view sizes: complex rows and K count twice.
    const int64_t Mr = CPLX ? 2 * p.M : p.M;
    const int64_t Kr = CPLX ? 2 * p.K : p.K;
    const int64_t i0 = (int64_t)tm * MT;  // real row offset of the tile
    const int64_t j0 = (int64_t)tn * NT;
    int64_t kend = Kr;
    if (TRI) {
        const int64_t lim = i0 + MT;  // real rows; K has the same (real) scale
        kend = lim < Kr ? lim : Kr;
    }
    const int nkt = (int)((kend + KT - 1) / KT);

    const R *Ar = reinterpret_cast<const R *>(p.A);
    const R *Br = reinterpret_cast<const R *>(p.Bm);
    const int64_t ldbr = CPLX ? 2 * p.ldb : p.ldb;

    // ---- global -> register staging ------------------------------------
    // A real: MT rows x KT cols, VEC rows per thread-load.
    constexpr int A_TPC = CPLX ? AROWS : MT / VEC;   // threads per column
    constexpr int A_CPP = 256 / A_TPC;               // columns per pass
    constexpr int A_PASSES = AK / A_CPP;
    static_assert(A_PASSES * A_CPP == AK, "A tile shape");
    // Bm: KT (real) rows x NT cols, VEC rows per thread-load.
    constexpr int B_TPC = KT / VEC;
    constexpr int B_CPP = 256 / B_TPC;
    constexpr int B_PASSES = NT / B_CPP;
    static_assert(B_PASSES * B_CPP == NT, "B tile shape");

    Vec ra[A_PASSES];
    Vec rb[B_PASSES];

    auto load_tiles = [&](int kt) {
        const int64_t k0 = (int64_t)kt * KT;  // real k offset
#pragma unroll
        for (int q = 0; q < A_PASSES; ++q) {
            const int flat = q * 256 + tid;
            const int kk = flat / A_TPC;
            const int rr = flat - kk * A_TPC;
            Vec v;
            if constexpr (CPLX) {
                const int64_t ic = i0 / 2 + rr;
                const int64_t kc = k0 / 2 + kk;
                v = Vec{0.0, 0.0};
                if (ic < p.M && kc < p.K) v = *reinterpret_cast<const Vec *>(Ar + 2 * (ic + kc * p.lda));
            } else {
                const int64_t i = i0 + (int64_t)rr * VEC;
                const int64_t k = k0 + kk;
                if (k < Kr && i + VEC <= Mr && p.a_vec) {
                    v = *reinterpret_cast<const Vec *>(Ar + i + k * p.lda);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        v[e] = (k < Kr && i + e < Mr) ? Ar[i + e + k * p.lda] : R(0);
                }
            }
            ra[q] = v;
        }
#pragma unroll
        for (int q = 0; q < B_PASSES; ++q) {
            const int flat = q * 256 + tid;
            const int jj = flat / B_TPC;
            const int kv = (flat - jj * B_TPC) * VEC;
            const int64_t j = j0 + jj;
            const int64_t k = k0 + kv;
            Vec v;
            if (j < p.N && k + VEC <= Kr && p.b_vec) {
                v = *reinterpret_cast<const Vec *>(Br + k + j * ldbr);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    v[e] = (j < p.N && k + e < Kr) ? Br[k + e + j * ldbr] : R(0);
            }
            rb[q] = v;
        }
    };

    auto store_tiles = [&](int buf) {
#pragma unroll
        for (int q = 0; q < A_PASSES; ++q) {
            const int flat = q * 256 + tid;
            const int kk = flat / A_TPC;
            const int rr = flat - kk * A_TPC;
            if constexpr (CPLX) {
                As[buf][kk][rr] = cplx{ra[q][0], ra[q][1]};
            } else {
                *reinterpret_cast<Vec *>(&As[buf][kk][rr * VEC]) = ra[q];
            }
        }
#pragma unroll
        for (int q = 0; q < B_PASSES; ++q) {
            const int flat = q * 256 + tid;
            const int jj = flat / B_TPC;
            const int kv = (flat - jj * B_TPC) * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) Bs[buf][kv + e][jj] = rb[q][e];
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = Acc{0, 0, 0, 0};

    // Complex A-fragment expansion constants (lane-fixed).
    // Real k' = 2*kc + ki follows the interleaved storage of Bm.  Real rows
    // are ordered so that the f64 MFMA result (row q + 4v in lane group q,
    // item v) holds the real and imaginary part of one complex row in items
    // (0, 1) and of another in items (2, 3): inside a 16-row MFMA tile, real
    // row t stands for complex row (t % 4) + 4 * (t / 8), part (t / 4) % 2.
    // Entry (row, k') of the embedded A is re if the parts agree, im for
    // (im row, re col) and -im for (re row, im col).
    const int t16 = lane & 15;
    const int a_crow = (t16 & 3) + 4 * (t16 >> 3);
    const int ri = (t16 >> 2) & 1;
    const int ki = (lane >> 4) & 1;
    const int a_part = (ri != ki) ? 1 : 0;
    const R a_sign = (ri == 0 && ki == 1) ? R(-1) : R(1);

    if (nkt > 0) {
        load_tiles(0);
        store_tiles(0);
        __syncthreads();
        for (int kt = 0; kt < nkt; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nkt) load_tiles(kt + 1);
#pragma unroll
            for (int ks = 0; ks < KT; ks += 4) {
                const int kr = ks + (lane >> 4);  // real k within the tile
                R af[FM], bf[FN];
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    if constexpr (CPLX) {
                        const int crow = (wm * WM + a * 16) / 2 + a_crow;  // complex row in tile
                        const cplx &z = As[buf][kr >> 1][crow];
                        af[a] = (a_part ? z.im : z.re) * a_sign;
                    } else {
                        af[a] = As[buf][kr][wm * WM + a * 16 + (lane & 15)];
                    }
                }
#pragma unroll
                for (int b = 0; b < FN; ++b) bf[b] = Bs[buf][kr][wn * WN + b * 16 + (lane & 15)];
#pragma unroll
                for (int a = 0; a < FM; ++a)
#pragma unroll
                    for (int b = 0; b < FN; ++b) acc[a][b] = Tr::mfma(af[a], bf[b], acc[a][b]);
            }
            if (kt + 1 < nkt) {
                store_tiles(buf ^ 1);
                __syncthreads();
            }
        }
    }

    // ---- epilogue: D = beta*C + gamma*acc ------------------------------
    // Item v of a lane in group q = lane/16 holds row Tr::out_row(q, v),
    // column lane % 16, of each 16 x 16 sub-tile.
    const int q = lane >> 4;
    const int cc = lane & 15;
    if constexpr (CPLX) {
        const cplx beta{p.beta.re, p.beta.im};
        const cplx gamma{p.gamma.re, p.gamma.im};
#pragma unroll
        for (int a = 0; a < FM; ++a) {
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int64_t j = j0 + wn * WN + b * 16 + cc;
                if (j >= p.N) continue;
                const int64_t cbase = (i0 + wm * WM + a * 16) / 2;  // first complex row
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t ic = cbase + q + 4 * h;
                    if (ic >= p.M) continue;
                    cplx z{acc[a][b][2 * h], acc[a][b][2 * h + 1]};
                    cplx out = Elem<cplx>::mul(gamma, z);
                    if (p.has_c) {
                        const cplx c = p.C[ic + j * p.ldc];
                        const cplx bc = Elem<cplx>::mul(beta, c);
                        out.re += bc.re;
                        out.im += bc.im;
                    }
                    if (ic < p.split) p.D2[ic + j * p.ldd2] = out;
                    else p.D[ic + j * p.ldd] = out;
                }
            }
        }
    } else {
        const R beta = (R)p.beta.re;
        const R gamma = (R)p.gamma.re;
#pragma unroll
        for (int a = 0; a < FM; ++a) {
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int64_t j = j0 + wn * WN + b * 16 + cc;
                if (j >= p.N) continue;
                const int64_t i = i0 + wm * WM + a * 16;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t ii = i + Tr::out_row(q, v);
                    if (ii >= p.M) continue;
                    R out = gamma * acc[a][b][v];
                    if (p.has_c) out = __builtin_fma(beta, p.C[ii + j * p.ldc], out);
                    if (ii < p.split) p.D2[ii + j * p.ldd2] = out;
                    else p.D[ii + j * p.ldd] = out;
                }
            }
        }
    }
}

template <typename T, int MT, int NT, int KT>
hipError_t launch_tile(const GemmDesc &g, hipStream_t st) {
    GemmParams<T> p;
    p.M = g.M;
    p.N = g.N;
    p.K = g.K;
    p.A = static_cast<const T *>(g.A);
    p.lda = g.lda;
    p.Bm = static_cast<const T *>(g.Bm);
    p.ldb = g.ldb;
    p.C = static_cast<const T *>(g.C);
    p.ldc = g.ldc;
    p.D = static_cast<T *>(g.D);
    p.ldd = g.ldd;
    p.D2 = static_cast<T *>(g.D2 ? g.D2 : g.D);
    p.ldd2 = g.D2 ? g.ldd2 : g.ldd;
    p.split = g.D2 ? g.split : 0;
    p.beta = g.beta;
    p.gamma = g.gamma;
    p.has_c = (g.C != nullptr) && (g.beta.re != 0.0 || g.beta.im != 0.0);
    constexpr int vecb = 16;
    const bool cplx_t = GemmTraits<T>::kCplx;
    p.a_vec = cplx_t ? 1
                     : ((reinterpret_cast<uintptr_t>(g.A) % vecb) == 0 &&
                        (g.lda * (int64_t)sizeof(T)) % vecb == 0);
    p.b_vec = cplx_t ? 1
                     : ((reinterpret_cast<uintptr_t>(g.Bm) % vecb) == 0 &&
                        (g.ldb * (int64_t)sizeof(T)) % vecb == 0);
    const int64_t Mr = cplx_t ? 2 * g.M : g.M;
    const int64_t tM = (Mr + MT - 1) / MT;
    const int64_t tN = (g.N + NT - 1) / NT;
    if (tM <= 0 || tN <= 0) return hipSuccess;
    if (tM * tN > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    p.tilesM = (int)tM;
    p.tilesN = (int)tN;
    if (g.a_lower)
        hipLaunchKernelGGL((gemm_kernel<T, MT, NT, KT, true>), dim3((unsigned)(tM * tN)), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((gemm_kernel<T, MT, NT, KT, false>), dim3((unsigned)(tM * tN)), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_launch(int dtype, const GemmDesc &g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    switch (dtype) {
        case R32F: return launch_tile<float, 128, 128, 32>(g, stream);
        case R64F: return launch_tile<double, 128, 128, 16>(g, stream);
        case C64F: return launch_tile<cplx, 128, 128, 16>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace trsm
