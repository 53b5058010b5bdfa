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
// Kernel families (launch_sized picks one by data type, shape and tile
// count; the rules and the measurements behind them are next to it):
//   * gemm_lf_kernel (fp64, complex fp64 through its real view) and
//     gemm_lf32_kernel (fp32, complex fp32): no LDS; each wave streams its own
//     A and Bm fragments into a ring of registers a few chunks of K ahead of
//     the MFMAs.  They take the single products whose tiles give the chip
//     enough waves (updates with 64 or more tiles of 128 x 128, triangular
//     solve products with 64 or more folded pairs), and the inversion's
//     larger batched doubling products;
//   * gemm_kernel: LDS-staged macro tiles (below), for the remaining shapes:
//     small and narrow products, unaligned operands, the inversion's small
//     batched products, split-K chunks;
//   * gemm_ks_kernel: fp64 and complex fp64 products with a long K and few
//     output tiles, K split over the waves of one workgroup;
//   * a product that splits K across workgroups (gemm_splitk_launch) runs
//     its chunks as one batched launch and adds them in a fixed order.
//
// gemm_kernel's gfx950 mapping:
//   * 256 threads = 2 x 2 wavefronts on a macro tile of MT x NT real rows x
//     columns (32 x 32 up to 128 x 128 by launch shape, see launch_sized);
//     each wave owns (MT/2) x (NT/2) as 16 x 16 tiles
//     of v_mfma_f64_16x16x4f64 (fp64, complex fp64) or
//     v_mfma_f32_16x16x4f32 (fp32: true fp32 products, no reduced-precision
//     splitting);
//   * global loads are raw buffer loads of 16 bytes per lane: reads past the
//     end of an operand return zero without a branch, and a K tile that
//     runs past K is zeroed by a select, so ragged shapes cost nothing in the
//     main loop;
//   * operands are staged through LDS, double-buffered: the loads of K tile
//     t+1 are in flight while the MFMAs of tile t run, one barrier per tile.
//     A is kept as [k][row] (its global layout) with an XOR swizzle of the
//     row index, Bm as [column][k] (its global layout too) with a padded
//     pitch, so that the fragment reads of the four lane groups spread over
//     all LDS banks;
//   * inside a K tile lane group q (lane / 16) works on k = q*KT/4 ... so
//     each lane's Bm fragments for consecutive MFMAs are adjacent in LDS and
//     come in 16-byte reads (the order of a sum over k is free);
//   * the rows fed to the A operand are permuted so that every lane ends
//     with runs of consecutive output rows: C is read and D written in
//     16-byte pieces;
//   * C is read at the start of a tile, straight into the accumulators
//     (acc = (beta/gamma) C, D = gamma acc), so its latency overlaps the
//     first operand loads instead of stalling the end of the tile;
//   * complex fp64 uses the real 2x2 embedding: a complex M x K by K x N
//     product is a real (2M x 2K) by (2K x N) product where each complex
//     a = ar + i ai of A becomes [[ar, -ai], [ai, ar]]; the interleaved
//     storage of Bm is already its real (2K x N) view, the A fragment is
//     expanded on the fly from the complex tile in LDS, and the real rows are
//     ordered so that each lane holds whole complex results.  This is exactly
//     the 4 real products per complex product (no 3M trick);
//   * with a triangular A the work of row tile i grows with i, so each
//     workgroup computes row tiles i and tilesM-1-i of one column tile, one
//     after the other: every workgroup gets the same amount of work;
//   * tiles are mapped so that each XCD (8 per chip, each with its own L2)
//     works on a band of 8 column tiles at a time, and the workgroups of one
//     XCD cover roughly 8 x 8 tiles, sharing the A and Bm panels in its L2;
//   * a product with few output tiles and a long K (a narrow B) can be cut
//     along K (gemm_splitk_launch): the chunks run as one batched launch
//     into partial sums, which a reduction kernel adds in a fixed order.
#include <cstdlib>
#include <type_traits>

#include "buffer_ops.h"
#include "scalar_ops.h"

namespace trsm {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef double d2v __attribute__((ext_vector_type(2)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));
template <typename T> struct GemmTraits;
template <> struct GemmTraits<float> {
    using R = float;
    using Acc = f4;
    static constexpr bool kCplx = false;
    __device__ __forceinline__ static Acc mfma(R a, R b, Acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // Row of a 16-row block fed by lane c of the A operand.  The f32 result
    // puts rows 4q .. 4q+3 in lane group q already.
    __device__ __forceinline__ static int a_row(int c) { return c; }
    __device__ __forceinline__ static int a_crow(int) { return 0; }  // complex only
    __device__ __forceinline__ static int a_ri(int) { return 0; }
};
template <> struct GemmTraits<double> {
    using R = double;
    using Acc = d4;
    static constexpr bool kCplx = false;
    __device__ __forceinline__ static Acc mfma(R a, R b, Acc c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    // The f64 result holds MFMA row q + 4v in item v of lane group q
    // (checked on gfx950); feeding row 4(c%4) + c/4 as MFMA row c turns that
    // into rows 4q .. 4q+3.
    __device__ __forceinline__ static int a_row(int c) { return 4 * (c & 3) + (c >> 2); }
    __device__ __forceinline__ static int a_crow(int) { return 0; }  // complex only
    __device__ __forceinline__ static int a_ri(int) { return 0; }
};
// Complex types: real row c of a 16-row MFMA block stands for complex row
// a_crow(c) of the block's 8, part a_ri(c) (0 re, 1 im), chosen so that
// with the result layout a lane holds complex rows 2q (items 0, 1) and
// 2q + 1 (items 2, 3) of lane group q.
template <> struct GemmTraits<cplx> {
    using R = double;
    using Acc = d4;
    static constexpr bool kCplx = true;
    __device__ __forceinline__ static Acc mfma(R a, R b, Acc c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static int a_row(int c) { return c; }
    // f64 result: row q + 4v in item v
    __device__ __forceinline__ static int a_crow(int c) { return 2 * (c & 3) + (c >> 3); }
    __device__ __forceinline__ static int a_ri(int c) { return (c >> 2) & 1; }
};
template <> struct GemmTraits<cplx32> {
    using R = float;
    using Acc = f4;
    static constexpr bool kCplx = true;
    __device__ __forceinline__ static Acc mfma(R a, R b, Acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static int a_row(int c) { return c; }
    // f32 result: row 4q + v in item v
    __device__ __forceinline__ static int a_crow(int c) { return c >> 1; }
    __device__ __forceinline__ static int a_ri(int c) { return c & 1; }
};

template <typename T>
struct GemmParams {
    int64_t M, N, K;  // in elements of T (complex counts for cplx)
    const T *A;
    int64_t lda, extA;  // extA: elements from A to one past the last one used
    const T *Bm;
    int64_t ldb, extB;
    const T *C;
    int64_t ldc;
    T *D;
    int64_t ldd;
    T *D2;
    int64_t ldd2;
    int64_t split;
    Scalar sc, gamma;  // accumulators start at sc * C; D = gamma * acc
    int has_c;
    int a_vec, b_vec;        // 16-byte aligned operand loads
    int c_vec, d_vec, d2_vec;  // 16-byte aligned C / D / D2 columns
    int tilesM, tilesN;
    int binner;  // batched launches (gridDim.y problems): see GemmDesc
    int64_t sAo, sAi, sBo, sBi, sCo, sCi, sDo, sDi;
    int64_t sKo;  // triangular A: column offset of problem zo in the triangle
    int fold;     // triangular A: one workgroup per pair of row tiles
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

// ---- C / D access in the accumulator layout -------------------------------
// Real types: a lane holds rows r .. r+3 (r % 4 == 0) of column j in items
// 0..3 of an accumulator.

template <typename R>
__device__ __forceinline__ void load_rows4(const R *X, int64_t ld, int64_t M, int64_t r, int64_t j,
                                           int vec, R out[4]) {
    const R *col = X + j * ld;
    if (vec && r + 3 < M) {
        if constexpr (sizeof(R) == 4) {
            const f4 v = *reinterpret_cast<const f4 *>(col + r);
            out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
        } else {
            const d2v v0 = *reinterpret_cast<const d2v *>(col + r);
            const d2v v1 = *reinterpret_cast<const d2v *>(col + r + 2);
            out[0] = v0[0]; out[1] = v0[1]; out[2] = v1[0]; out[3] = v1[1];
        }
    } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) out[v] = (r + v < M) ? col[r + v] : R(0);
    }
}

template <typename R>
__device__ __forceinline__ void store_rows4(R *X, int64_t ld, int64_t lim, int64_t r, int64_t j,
                                            int vec, const R in[4]) {
    R *col = X + j * ld;
    if (vec && r + 3 < lim) {
        if constexpr (sizeof(R) == 4) {
            *reinterpret_cast<f4 *>(col + r) = f4{in[0], in[1], in[2], in[3]};
        } else {
            *reinterpret_cast<d2v *>(col + r) = d2v{in[0], in[1]};
            *reinterpret_cast<d2v *>(col + r + 2) = d2v{in[2], in[3]};
        }
    } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (r + v < lim) col[r + v] = in[v];
    }
}

// TRI: A is lower triangular (the solve GEMM); a separate instantiation so
// that the solve and the update appear as distinct kernels in traces.
// VEC: A and Bm columns are 16-byte aligned (16-byte loads); otherwise the
// loads are split into dwords.
// BLO: Bm is lower triangular (explicit zeros above its diagonal), as the
// right factor of the inversion's second product: a column tile starting at
// column j0 skips the K tiles wholly above row j0.
// WIDE: A and Bm are read through 64-bit global addresses (ld16_wide) instead
// of 32-bit buffer offsets, for leading dimensions so large that the offsets
// inside one tile would not fit (fp64: lda beyond about 8 M elements, or ldb
// beyond about 2 M on the widest tile); only the 64 x 32 tile has this form.
template <typename T, int MT, int NT, int KT, bool TRI, bool VEC, bool BLO = false, bool WIDE = false>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams<T> p) {
    using Tr = GemmTraits<T>;
    using R = typename Tr::R;
    using Acc = typename Tr::Acc;
    constexpr bool CPLX = Tr::kCplx;
    constexpr int VR = 16 / (int)sizeof(R);  // reals per 16-byte load
    constexpr int WM = MT / 2, WN = NT / 2;  // per-wave tile (real rows x cols)
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int KS = KT / 4;  // k values of one lane group inside a K tile
    constexpr int CW = VR;      // k values per 16-byte Bm fragment read
    static_assert(KS % CW == 0, "K tile");
    // A tile: AK columns x AR rows of T (complex: complex rows and k).
    constexpr int AK = CPLX ? KT / 2 : KT;
    constexpr int AR = CPLX ? MT / 2 : MT;
    constexpr int AU = 16 / (int)sizeof(T);  // elements of T per 16-byte load
    constexpr int SA = AR + 4;         // row pitch (16-byte multiple)
    // Swizzle of the A tile.  Lane group q reads k rows [q*KPG, q*KPG + KPG)
    // of the tile, and with any 16-byte pitch those start 0 or 32 banks
    // apart, so groups 0 and 2 (1 and 3) hit the same banks.  Row r of k
    // row kk is stored at r ^ swz(kk): 16 dwords further in every other
    // pair of groups, which puts the four groups on four distinct sets of
    // 16 banks; the XOR keeps each 16-byte store contiguous.
    constexpr int KPG = CPLX ? KS / 2 : KS;  // A-tile k rows per lane group
    constexpr int SW = 64 / (int)sizeof(T);  // elements in 16 dwords
    static_assert(AR >= 2 * SW && SW % AU == 0, "A swizzle");
    constexpr int SB = KT + (VR == 4 ? 4 : 2);  // 36 (f32) / 18 (f64) reals: 9 x 16 bytes
    __shared__ __attribute__((aligned(16))) T As[2][AK][SA];
    __shared__ __attribute__((aligned(16))) R Bs[2][NT][SB];
    const auto a_swz = [](int kk) { return ((kk / KPG) & 1) * SW; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int c16 = lane & 15;
    const int q = lane >> 4;

    // triangular A: workgroup w takes row tiles i and tilesM-1-i of one
    // column tile (their K ranges sum to the same length for every i).  A
    // column slice of the triangle (split K) is not folded: most of its row
    // tiles have the slice's full length.
    const bool fold = TRI && p.fold;
    const int rowsM = fold ? (p.tilesM + 1) / 2 : p.tilesM;
    if (blockIdx.x >= (unsigned)(rowsM * p.tilesN)) return;
    // Operands of problem blockIdx.y of a batch.  Kept in locals: `p` is
    // never written, so its fields stay scalar (kernel-argument) loads.
    const int zo = (int)blockIdx.y / p.binner;
    const int zi = (int)blockIdx.y - zo * p.binner;
    const T *__restrict__ pA = p.A + (zo * p.sAo + zi * p.sAi);
    const T *__restrict__ pB = p.Bm + (zo * p.sBo + zi * p.sBi);
    const T *__restrict__ pC = p.C + (zo * p.sCo + zi * p.sCi);
    T *__restrict__ pD = p.D + (zo * p.sDo + zi * p.sDi);
    T *__restrict__ pD2 = p.D2 + (zo * p.sDo + zi * p.sDi);
    int tm0, tn;
    map_tile(blockIdx.x, rowsM, p.tilesN, tm0, tn);

    // one pass per row tile: tm0, then (triangular A) its partner
    const int tm1 = p.tilesM - 1 - tm0;
    const int npass = (fold && tm1 != tm0) ? 2 : 1;
    for (int pass = 0; pass < npass; ++pass) {
        const int tm = pass == 0 ? tm0 : tm1;
        if (pass > 0) __syncthreads();  // the LDS buffers are reused
        const int64_t Kr = CPLX ? 2 * p.K : p.K;  // real K
        const int64_t i0 = (int64_t)tm * MT;      // real row offset of the tile
        const int64_t j0 = (int64_t)tn * NT;
        const int64_t i0t = CPLX ? i0 / 2 : i0;
        int64_t kend = Kr;
        if (TRI) {
            // real rows; K has the same (real) scale.  Problem zo of a batch
            // starts zo*sKo columns right of the triangle's first column.
            const int64_t koff = (int64_t)zo * p.sKo * (CPLX ? 2 : 1);
            const int64_t lim = i0 + MT - koff;
            kend = lim < Kr ? lim : Kr;
            if (kend < 0) kend = 0;
        }
        // lower-triangular Bm: its rows above j0 are zero in this column tile
        const int ktb = BLO ? (int)((CPLX ? 2 * j0 : j0) / KT) : 0;
        const int nkt = (int)((kend + KT - 1) / KT) - ktb;

        // ---- accumulators start at sc * C ----------------------------------
        Acc acc[FM][FN];
        if (p.has_c) {
            if constexpr (CPLX) {
                const T sc = Elem<T>::from(p.sc);
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    const int64_t cb = (i0 + wm * WM + a * 16) / 2 + 2 * q;  // complex rows cb, cb+1
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        const int64_t j = j0 + wn * WN + b * 16 + c16;
                        T z0 = Elem<T>::zero(), z1 = Elem<T>::zero();
                        if (j < p.N) {
                            if (cb < p.M) z0 = Elem<T>::mul(sc, pC[cb + j * p.ldc]);
                            if (cb + 1 < p.M) z1 = Elem<T>::mul(sc, pC[cb + 1 + j * p.ldc]);
                        }
                        acc[a][b] = Acc{z0.re, z0.im, z1.re, z1.im};
                    }
                }
            } else {
                const R sc = (R)p.sc.re;
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    const int64_t r = i0 + wm * WM + a * 16 + 4 * q;
#pragma unroll
                    for (int b = 0; b < FN; ++b) {
                        const int64_t j = j0 + wn * WN + b * 16 + c16;
                        R cv[4] = {R(0), R(0), R(0), R(0)};
                        if (j < p.N) load_rows4<R>(pC, p.ldc, p.M, r, j, p.c_vec, cv);
                        acc[a][b] = Acc{sc * cv[0], sc * cv[1], sc * cv[2], sc * cv[3]};
                    }
                }
            }
        } else {
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b) acc[a][b] = Acc{0, 0, 0, 0};
        }

        // ---- global -> register staging ------------------------------------
        constexpr int A_TPC = AR / AU;  // threads per A column
        constexpr int A_CPP = 256 / A_TPC;
        constexpr int A_PASSES = AK / A_CPP;
        static_assert(A_PASSES * A_CPP == AK, "A tile shape");
        constexpr int B_TPC = KT / VR;  // threads per Bm column (real view)
        constexpr int B_CPP = 256 / B_TPC;
        constexpr int B_PASSES = NT / B_CPP;
        static_assert(B_PASSES * B_CPP == NT, "B tile shape");
        constexpr int DW = (int)sizeof(R) / 4;  // dwords per real

        // Register staging sets: with DEPTH 2 the loads of tile kt+2 are in
        // flight while tile kt+1 waits in the other set, so a load has two
        // tiles of products to arrive.  Small tiles run few products per K
        // tile and need that.  The fp64 128 x 64 tile keeps one set: a second
        // one takes it from 168 to 194 VGPRs, three waves per SIMD to two,
        // and measured slower (fp64 8192^2 9.77 -> 9.80 ms).  The complex
        // 64 x 128 tile stays at three waves with two sets and gains
        // (complex 8192 x 2048 9.83 -> 9.55 ms; complex fp32 5.06 -> 4.85).
        constexpr int DEPTH = (MT * NT <= 64 * 64 || CPLX) ? 2 : 1;
        u4v ra[DEPTH][A_PASSES];
        u4v rb[DEPTH][B_PASSES];

        // Loads of K tile kt into registers.  The ragged-K mask is applied when
        // the registers are written to LDS (store_tiles), not here: a select on
        // the loaded values would make the compiler wait for the loads right
        // after issuing them, before the MFMAs they are meant to overlap.
        // A tile past the last one (live == false) is still issued, on an
        // empty range: its loads touch no memory and return zero.  Issuing
        // the same loads on every path lets the compiler wait for exactly the
        // tile it stores next; with the prefetch under a branch it waited for
        // every load in flight, the prefetch just issued included.
        auto load_tiles = [&](int kt, auto set_c, bool live = true) {
            constexpr int S = decltype(set_c)::value;
            const int64_t k0 = (int64_t)(kt + ktb) * KT;  // real k offset
            const int64_t k0t = CPLX ? k0 / 2 : k0;
            {
                const int64_t off = i0t + k0t * p.lda;
                const int64_t lim = live ? (p.extA - off) * (int64_t)sizeof(T) : 0;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(pA + off, WIDE ? 0 : lim);
#pragma unroll
                for (int s = 0; s < A_PASSES; ++s) {
                    const int flat = s * 256 + tid;
                    const int kk = flat / A_TPC;
                    const int rr = flat - kk * A_TPC;
                    const int64_t boff = ((int64_t)rr * AU + (int64_t)kk * p.lda) * (int64_t)sizeof(T);
                    if constexpr (WIDE)
                        ra[S][s] = ld16_wide(reinterpret_cast<const char *>(pA + off), boff, lim);
                    else
                        ra[S][s] = ld16<VEC>(rs, (uint32_t)boff);
                }
            }
            {
                const int64_t off = k0t + j0 * p.ldb;
                const int64_t lim = live ? (p.extB - off) * (int64_t)sizeof(T) : 0;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(pB + off, WIDE ? 0 : lim);
#pragma unroll
                for (int s = 0; s < B_PASSES; ++s) {
                    const int flat = s * 256 + tid;
                    const int jj = flat / B_TPC;
                    const int kv = (flat - jj * B_TPC) * VR;  // real k inside the tile
                    const int64_t kvt = CPLX ? kv / 2 : kv;
                    const int64_t boff = (kvt + (int64_t)jj * p.ldb) * (int64_t)sizeof(T);
                    if constexpr (WIDE)
                        rb[S][s] = ld16_wide(reinterpret_cast<const char *>(pB + off), boff, lim);
                    else
                        rb[S][s] = ld16<VEC>(rs, (uint32_t)boff);
                }
            }
        };

        // Registers of K tile kt -> LDS buffer buf; entries with k >= K become
        // zero (only the last, ragged K tile has any: a uniform test first).
        auto store_tiles = [&](int buf, int kt, auto set_c) {
            constexpr int S = decltype(set_c)::value;
            const int64_t k0 = (int64_t)(kt + ktb) * KT;
            const int64_t k0t = CPLX ? k0 / 2 : k0;
            const bool ragged = k0 + KT > Kr;  // wave-uniform
#pragma unroll
            for (int s = 0; s < A_PASSES; ++s) {
                const int flat = s * 256 + tid;
                const int kk = flat / A_TPC;
                const int rr = flat - kk * A_TPC;
                u4v v = ra[S][s];
                if (ragged && k0t + kk >= p.K) v = u4v{0u, 0u, 0u, 0u};
                *reinterpret_cast<u4v *>(&As[buf][kk][(rr * AU) ^ a_swz(kk)]) = v;
            }
#pragma unroll
            for (int s = 0; s < B_PASSES; ++s) {
                const int flat = s * 256 + tid;
                const int jj = flat / B_TPC;
                const int kv = (flat - jj * B_TPC) * VR;
                u4v v = rb[S][s];
                if (ragged) {
#pragma unroll
                    for (int e = 0; e < VR; ++e)
                        if (k0 + kv + e >= Kr)
#pragma unroll
                            for (int d = 0; d < DW; ++d) v[e * DW + d] = 0u;
                }
                *reinterpret_cast<u4v *>(&Bs[buf][jj][kv]) = v;
            }
        };

        // Complex A-fragment expansion (lane-fixed part).  Real row t = c16 of a
        // 16-row block stands for complex row 2(t % 4) + t / 8 of the block's 8,
        // part (t / 4) % 2; with the f64 result layout (row q + 4v in item v) a
        // lane then holds complex rows 2q (items 0, 1) and 2q + 1 (items 2, 3).
        const int a_crow = CPLX ? Tr::a_crow(c16) : 0;
        const int a_ri = CPLX ? Tr::a_ri(c16) : 0;
        const int a_row = Tr::a_row(c16);

        // Products of the K tile in LDS buffer buf.
        auto mfma_tile = [&](const int buf) {
#pragma unroll
            for (int s0 = 0; s0 < KS; s0 += CW) {
                const int kb = q * KS + s0;  // real k of this chunk inside the tile
                R bf[FN][CW];
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const u4v v = *reinterpret_cast<const u4v *>(&Bs[buf][wn * WN + b * 16 + c16][kb]);
                    if constexpr (sizeof(R) == 4) {
                        const f4 fv = __builtin_bit_cast(f4, v);
#pragma unroll
                        for (int e = 0; e < CW; ++e) bf[b][e] = fv[e];
                    } else {
                        const d2v dv = __builtin_bit_cast(d2v, v);
                        bf[b][0] = dv[0];
                        bf[b][1] = dv[1];
                    }
                }
                R af[FM][CW];
#pragma unroll
                for (int a = 0; a < FM; ++a) {
                    if constexpr (CPLX) {
                        // real k = kb + e: complex k (kb + e) / 2, part e % 2 (kb even)
#pragma unroll
                        for (int e2 = 0; e2 < CW / 2; ++e2) {
                            const int kc = (kb >> 1) + e2;
                            const T z = As[buf][kc][((wm * WM + a * 16) / 2 + a_crow) ^ a_swz(kc)];
                            af[a][2 * e2] = a_ri ? z.im : z.re;       // k part 0
                            af[a][2 * e2 + 1] = a_ri ? z.re : -z.im;  // k part 1
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < CW; ++e)
                            af[a][e] = As[buf][kb + e][(wm * WM + a * 16 + a_row) ^ a_swz(kb + e)];
                    }
                }
#pragma unroll
                for (int e = 0; e < CW; ++e)
#pragma unroll
                    for (int a = 0; a < FM; ++a)
#pragma unroll
                        for (int b = 0; b < FN; ++b) acc[a][b] = Tr::mfma(af[a][e], bf[b][e], acc[a][b]);
            }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        if (nkt > 0) {
            if constexpr (DEPTH == 2) {
                load_tiles(0, I0{});
                load_tiles(1, I1{}, nkt > 1);
                store_tiles(0, 0, I0{});
                __syncthreads();
                // step kt (kt % 2 == S): set S held tile kt (already in LDS)
                // and takes tile kt+2; tile kt+1 goes from set S^1 to buffer S^1
                auto step = [&](int kt, auto set_c) {
                    constexpr int S = decltype(set_c)::value;
                    using IN = std::integral_constant<int, S ^ 1>;
                    load_tiles(kt + 2, set_c, kt + 2 < nkt);
                    mfma_tile(S);
                    if (kt + 1 < nkt) {
                        store_tiles(S ^ 1, kt + 1, IN{});
                        __syncthreads();
                    }
                };
                for (int kt = 0; kt < nkt; kt += 2) {
                    step(kt, I0{});
                    if (kt + 1 < nkt) step(kt + 1, I1{});
                }
            } else {
                load_tiles(0, I0{});
                store_tiles(0, 0, I0{});
                __syncthreads();
                for (int kt = 0; kt < nkt; ++kt) {
                    const int buf = kt & 1;
                    if (kt + 1 < nkt) load_tiles(kt + 1, I0{});
                    mfma_tile(buf);
                    if (kt + 1 < nkt) {
                        store_tiles(buf ^ 1, kt + 1, I0{});
                        __syncthreads();
                    }
                }
            }
        }

        // ---- epilogue: D = gamma * acc, rows below `split` to D2 --------------
        if constexpr (CPLX) {
            const T gamma = Elem<T>::from(p.gamma);
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int64_t cb = (i0 + wm * WM + a * 16) / 2 + 2 * q;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int64_t j = j0 + wn * WN + b * 16 + c16;
                    if (j >= p.N) continue;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int64_t ic = cb + h;
                        if (ic >= p.M) continue;
                        const T out = Elem<T>::mul(gamma, T{acc[a][b][2 * h], acc[a][b][2 * h + 1]});
                        if (ic < p.split) pD2[ic + j * p.ldd2] = out;
                        else pD[ic + j * p.ldd] = out;
                    }
                }
            }
        } else {
            const R gamma = (R)p.gamma.re;
#pragma unroll
            for (int a = 0; a < FM; ++a) {
                const int64_t r = i0 + wm * WM + a * 16 + 4 * q;
                if (r >= p.M) continue;
#pragma unroll
                for (int b = 0; b < FN; ++b) {
                    const int64_t j = j0 + wn * WN + b * 16 + c16;
                    if (j >= p.N) continue;
                    R out[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) out[v] = gamma * acc[a][b][v];
                    if (r + 3 < p.split) {
                        store_rows4<R>(pD2, p.ldd2, p.M, r, j, p.d2_vec, out);
                    } else if (r >= p.split) {
                        store_rows4<R>(pD, p.ldd, p.M, r, j, p.d_vec, out);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int64_t ii = r + v;
                            if (ii >= p.M) break;
                            if (ii < p.split) pD2[ii + j * p.ldd2] = out[v];
                            else pD[ii + j * p.ldd] = out[v];
                        }
                    }
                }
            }
        }
    }  // pass
}

// ---- fp64 products without LDS ---------------------------------------------
// A v_mfma_f64_16x16x4f64 holds the matrix core of its SIMD for 64 cycles, so
// on gfx950 the fp64 operands are cheap next to the arithmetic, and the
// shared-LDS pipeline of gemm_kernel loses its time at the K-tile boundaries
// (the wait for the next tile, the LDS hand-off, the barrier), with two
// waves per SIMD to hide it.  gemm_lf_kernel has neither LDS nor barriers:
// each wave computes 64 x 64 outputs of its workgroup's 128 x 128 tile and
// streams its own rows of A and columns of Bm from memory (mostly L2) into a
// ring of registers, RING chunks of 8 k ahead of the products that use them.
//   * A: lane (c, q) (c = lane % 16, q = lane / 16) loads rows 2c, 2c + 1
//     and 32 + 2c, 33 + 2c of the wave's 64 at chunk k = 2q + s (s = 0, 1),
//     16 bytes each, consecutive lanes on consecutive rows; MFMA row tile a
//     takes row 2c + (a & 1) + 32 (a >> 1) as its row c;
//   * Bm: lane (c, q) loads k = 2q, 2q + 1 of columns c + 16b (b = 0..3),
//     16 bytes each; k index q of MFMA step s is chunk k 2q + s on both
//     sides (the order of a sum over k is free);
//   * the f64 result puts MFMA row q + 4v in item v of lane group q, so a
//     lane holds output rows 2(q + 4v), 2(q + 4v) + 1 (tiles 0, 1) and 32
//     rows further (tiles 2, 3): C and D move in 16-byte pairs;
//   * loads are raw buffer loads rebased per chunk: a read past the end of
//     an operand returns zero, and the ragged last chunk (K % 8) gives the
//     lanes whose k is past K an offset out of range, so A and Bm both read
//     zero there (whatever the memory past K holds).
// Measured on MI355X against the 128 x 128 gemm_kernel tile, fp64
// 1024 x 8192 updates: 68.3 against 64.5 TFLOP/s at K = 7168, 67.7 against
// 63.9 at K = 4096, 64.9 against 59.3 at K = 1024.
// NBT: 16-column MFMA tiles per wave (4: 64 x 64 per wave, the workgroup a
// 2 x 2 grid of waves on 128 x 128; 2: 64 x 32 per wave, the workgroup four
// waves side by side on 64 x 128).
// TRI: A is lower triangular with explicit zeros above the diagonal (the
// diagonal-block solve, M == K): a 64-row tile at r0 needs K up to r0 + 64
// only; each wave takes row tiles i and T-1-i (T = 64-row tiles) one after
// the other, so every wave gets the same length of K (no barriers: waves
// run independently).
// CPLX: complex fp64 through the real 2 x 2 embedding (each complex a of A
// is [[ar, -ai], [ai, ar]]).  p describes the real view: M and K count real
// rows and real k (twice the complex counts), Bm, C, D and D2 are their
// interleaved storage read as real with doubled leading dimensions, split
// counts real rows; only A keeps complex addressing (lda in complex elements,
// extA in doubles).  One 16-byte load of complex A(i, k) gives lane (c, q)
// the whole 2 x 2 block it feeds for complex row i: (ar, ai) on step s = 0,
// (-ai, ar) on s = 1; a pair of output rows is one complex element, so C is
// scaled by sc and the result by gamma as complex numbers.
// BAT: batched launches, problem blockIdx.y (as gemm_kernel).  BLO: Bm is
// lower triangular with explicit zeros above its diagonal (the inversion's
// second product): a wave's K loop starts at its first column.
template <int RING, int NBT, bool TRI, bool CPLX = false, bool BAT = false, bool BLO = false>
__global__ __launch_bounds__(256, 2) void gemm_lf_kernel(GemmParams<double> p) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform (the buffer resources below are built from it and must
    // be scalar values)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15;
    const int q = lane >> 4;
    int tm, tn;
    map_tile(blockIdx.x, p.tilesM, p.tilesN, tm, tn);
    const int zo = BAT ? (int)blockIdx.y / p.binner : 0;
    const int zi = BAT ? (int)blockIdx.y - zo * p.binner : 0;
    const double *__restrict__ pA = p.A + (zo * p.sAo + zi * p.sAi);
    const double *__restrict__ pB = p.Bm + (zo * p.sBo + zi * p.sBi);
    // C, D and D2 of the problem, formed where they are used
    auto cptr = [&]() -> const double * {
        if constexpr (BAT) return p.C + (zo * p.sCo + zi * p.sCi);
        else return p.C;
    };
    auto dptr = [&](double *base) -> double * {
        if constexpr (BAT) return base + (zo * p.sDo + zi * p.sDi);
        else return base;
    };
    const int64_t lda = p.lda, ldb = p.ldb;
    // real: rows 2c, 2c + 1 at k = 2q (offA0) and 2q + 1 (offA1), 32 rows
    // further at +256 bytes; complex: element (c, q) and 16 complex rows
    // further (+256 bytes)
    const uint32_t offA0 = CPLX ? (uint32_t)((c16 + q * lda) * 16) : (uint32_t)((2 * c16 + 2 * q * lda) * 8);
    const uint32_t offA1 = offA0 + (uint32_t)(lda * 8);
    uint32_t offB[NBT];
#pragma unroll
    for (int b = 0; b < NBT; ++b) offB[b] = (uint32_t)((2 * q + (c16 + 16 * (int64_t)b) * ldb) * 8);
    const double sc = p.sc.re, gamma = p.gamma.re;
    const double sci = p.sc.im, gammai = p.gamma.im;  // complex only

    // the wave's output block: rows [r0, r0 + 64), columns [c0, c0 + 16 NBT),
    // products over k in [kb, K) (kb a multiple of 8)
    auto run_tile = [&](const int64_t r0, const int64_t c0, const int64_t kb, const int64_t K) {
        // ---- accumulators start at sc * C ------------------------------------
        d4 acc[4][NBT];
#pragma unroll
        for (int b = 0; b < NBT; ++b) {
            const int64_t j = c0 + c16 + 16 * b;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t rr = r0 + 2 * (q + 4 * v);
                double x[4] = {0.0, 0.0, 0.0, 0.0};
                if (p.has_c && j < p.N) {
                    const double *col = cptr() + j * p.ldc;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {  // rows rr (tiles 0, 1) and rr + 32 (tiles 2, 3)
                        const int64_t r = rr + 32 * h;
                        if (p.c_vec && r + 1 < p.M) {
                            const d2v c2 = *reinterpret_cast<const d2v *>(col + r);
                            x[2 * h] = c2[0];
                            x[2 * h + 1] = c2[1];
                        } else {
                            if (r < p.M) x[2 * h] = col[r];
                            if (r + 1 < p.M) x[2 * h + 1] = col[r + 1];
                        }
                    }
                }
                if constexpr (CPLX) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {  // complex sc * C
                        acc[2 * h][b][v] = sc * x[2 * h] - sci * x[2 * h + 1];
                        acc[2 * h + 1][b][v] = sc * x[2 * h + 1] + sci * x[2 * h];
                    }
                } else {
#pragma unroll
                    for (int a = 0; a < 4; ++a) acc[a][b][v] = sc * x[a];
                }
            }
        }

        // ---- operand ring -----------------------------------------------------
        d2v ra[RING][4], rb[RING][NBT];
        // chunk [k0, k0 + 8) into ring slot `slot`; live == false issues the
        // loads on an empty range (no memory access, zeros)
        auto load = [&](int slot, int64_t k0, bool live) {
            // complex: element (r0/2, k0/2) sits at double offset r0 + k0 lda
            const int64_t oa = r0 + k0 * lda;
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(pA + oa, live ? (p.extA - oa) * 8 : 0);
            ra[slot][0] = __builtin_bit_cast(d2v, ld16<true>(rsa, offA0));
            ra[slot][1] = __builtin_bit_cast(d2v, ld16<true>(rsa, offA0 + 256));
            if constexpr (!CPLX) {
                ra[slot][2] = __builtin_bit_cast(d2v, ld16<true>(rsa, offA1));
                ra[slot][3] = __builtin_bit_cast(d2v, ld16<true>(rsa, offA1 + 256));
            }
            const int64_t ob = k0 + c0 * ldb;
            const __amdgpu_buffer_rsrc_t rsb = make_rsrc(pB + ob, live ? (p.extB - ob) * 8 : 0);
#pragma unroll
            for (int b = 0; b < NBT; ++b) rb[slot][b] = __builtin_bit_cast(d2v, ld16<true>(rsb, offB[b]));
        };
        auto compute = [&](const d2v (&a4)[4], const d2v (&bq)[NBT]) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                double av[4];
                if constexpr (CPLX) {
                    if (s == 0) {
                        av[0] = a4[0][0]; av[1] = a4[0][1]; av[2] = a4[1][0]; av[3] = a4[1][1];
                    } else {
                        av[0] = -a4[0][1]; av[1] = a4[0][0]; av[2] = -a4[1][1]; av[3] = a4[1][0];
                    }
                } else {
                    av[0] = a4[2 * s][0]; av[1] = a4[2 * s][1]; av[2] = a4[2 * s + 1][0]; av[3] = a4[2 * s + 1][1];
                }
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < NBT; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bq[b][s], acc[a][b], 0, 0, 0);
            }
        };
        const int64_t nkf = (K - kb) / 8;  // full chunks
#pragma unroll
        for (int u = 0; u < RING; ++u) load(u, kb + 8 * u, u < nkf);
        // Whole rounds of RING chunks with no condition around the products
        // and loads, then the last chunks (already loaded): a condition per
        // slot in the loop gave the wait counters a path on which the later
        // slots' loads were not issued, and the loop head then waited for
        // every load in flight once per round.
        int64_t kc = 0;
        for (; kc + RING <= nkf; kc += RING) {
#pragma unroll
            for (int u = 0; u < RING; ++u) {
                compute(ra[u], rb[u]);
                load(u, kb + 8 * (kc + u + RING), kc + u + RING < nkf);
            }
        }
#pragma unroll
        for (int u = 0; u < RING; ++u)
            if (kc + u < nkf) compute(ra[u], rb[u]);  // uniform
        // ragged last chunk: k = 8 nkf + 2q + s exists only while below K; the
        // lanes past it read zero from A and Bm (8-byte Bm loads, so a pair
        // straddling K keeps its first element)
        const int kr = (int)(K - kb - 8 * nkf);
        if (kr > 0) {
            const int64_t k0 = kb + 8 * nkf;
            const int64_t oa = r0 + k0 * lda;
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(pA + oa, (p.extA - oa) * 8);
            const uint32_t dead = 0xfffffff0u;
            const bool ok0 = 2 * q < kr, ok1 = 2 * q + 1 < kr;
            d2v ta[4], tb[NBT];
            ta[0] = __builtin_bit_cast(d2v, ld16<true>(rsa, ok0 ? offA0 : dead));
            ta[1] = __builtin_bit_cast(d2v, ld16<true>(rsa, ok0 ? offA0 + 256 : dead));
            const int64_t ob = k0 + c0 * ldb;
            const __amdgpu_buffer_rsrc_t rsb = make_rsrc(pB + ob, (p.extB - ob) * 8);
            if constexpr (CPLX) {
                // the real K is even: a complex k is whole or absent
#pragma unroll
                for (int b = 0; b < NBT; ++b) tb[b] = __builtin_bit_cast(d2v, ld16<true>(rsb, ok0 ? offB[b] : dead));
            } else {
                ta[2] = __builtin_bit_cast(d2v, ld16<true>(rsa, ok1 ? offA1 : dead));
                ta[3] = __builtin_bit_cast(d2v, ld16<true>(rsa, ok1 ? offA1 + 256 : dead));
#pragma unroll
                for (int b = 0; b < NBT; ++b) {
                    const u2v lo = __builtin_amdgcn_raw_buffer_load_b64(rsb, ok0 ? offB[b] : dead, 0, 0);
                    const u2v hi = __builtin_amdgcn_raw_buffer_load_b64(rsb, ok1 ? offB[b] + 8 : dead, 0, 0);
                    tb[b] = d2v{__builtin_bit_cast(double, lo), __builtin_bit_cast(double, hi)};
                }
            }
            compute(ta, tb);
        }

        // ---- epilogue: D = gamma * acc, rows below `split` to D2 ----------------
#pragma unroll
        for (int b = 0; b < NBT; ++b) {
            const int64_t j = c0 + c16 + 16 * b;
            if (j >= p.N) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t r = r0 + 2 * (q + 4 * v) + 32 * h;
                    if (r >= p.M) continue;
                    double x0, x1;
                    if constexpr (CPLX) {  // complex gamma * acc
                        x0 = gamma * acc[2 * h][b][v] - gammai * acc[2 * h + 1][b][v];
                        x1 = gamma * acc[2 * h + 1][b][v] + gammai * acc[2 * h][b][v];
                    } else {
                        x0 = gamma * acc[2 * h][b][v];
                        x1 = gamma * acc[2 * h + 1][b][v];
                    }
                    if (r + 1 < p.M && r + 1 < p.split) {
                        double *dst = dptr(p.D2) + j * p.ldd2 + r;
                        if (p.d2_vec) *reinterpret_cast<d2v *>(dst) = d2v{x0, x1};
                        else { dst[0] = x0; dst[1] = x1; }
                    } else if (r + 1 < p.M && r >= p.split) {
                        double *dst = dptr(p.D) + j * p.ldd + r;
                        if (p.d_vec) *reinterpret_cast<d2v *>(dst) = d2v{x0, x1};
                        else { dst[0] = x0; dst[1] = x1; }
                    } else {
                        if (r < p.split) dptr(p.D2)[r + j * p.ldd2] = x0;
                        else dptr(p.D)[r + j * p.ldd] = x0;
                        if (r + 1 < p.M) {
                            if (r + 1 < p.split) dptr(p.D2)[r + 1 + j * p.ldd2] = x1;
                            else dptr(p.D)[r + 1 + j * p.ldd] = x1;
                        }
                    }
                }
            }
        }
    };

    if constexpr (TRI) {
        // tm: pair of 64-row tiles (tm, T-1-tm); the wave's 16 NBT columns
        const int T = (int)((p.M + 63) / 64);
        const int64_t c0 = (int64_t)tn * 64 * NBT + (int64_t)wave * 16 * NBT;
        const int t1 = T - 1 - tm;
        for (int pass = 0; pass < (t1 != tm ? 2 : 1); ++pass) {
            const int64_t r0 = (int64_t)(pass == 0 ? tm : t1) * 64;
            run_tile(r0, c0, 0, r0 + 64 < p.K ? r0 + 64 : p.K);
        }
    } else {
        const int64_t r0 = (int64_t)tm * 128 + (wave & 1) * 64;
        const int64_t c0 = (int64_t)tn * 32 * NBT + (int64_t)(wave >> 1) * 16 * NBT;
        // lower-triangular Bm: its rows above c0 are zero in these columns
        if constexpr (BLO) {
            // the K range of column block t shrinks with t: each workgroup
            // takes blocks t and TN-1-t, one after the other, so every
            // workgroup gets the same length of K (complex: real k 2j starts
            // complex column j)
            const int TN = (int)((p.N + 32 * NBT - 1) / (32 * NBT));
            const int tn1 = TN - 1 - tn;
            for (int pass = 0; pass < (tn1 != tn ? 2 : 1); ++pass) {
                const int64_t cp = (int64_t)(pass == 0 ? tn : tn1) * 32 * NBT + (int64_t)(wave >> 1) * 16 * NBT;
                const int64_t kb = (CPLX ? 2 : 1) * cp;
                run_tile(r0, cp, kb < p.K ? kb : p.K, p.K);
            }
        } else {
            run_tile(r0, c0, 0, p.K);
        }
    }
}

// ---- fp64 products split along K inside one workgroup --------------------
// A narrow B gives the blocked path's products few output tiles and a long
// K (fp64 8192 x 64 at IB 1024: a 7168 x 64 update with K = 1024, 1024 x 64
// triangular solves with K up to 1024).  The split-K form (a batch of
// partial products, then a reduction kernel) pays a second launch and
// writes and reads its partial sums through memory.  gemm_ks_kernel keeps
// the split inside one workgroup: its KW waves compute the same 64 x 16
// output tile, wave w over the w-th of KW equal runs of 8-k chunks (the
// fragment layout of gemm_lf_kernel with one column tile), then waves 1 ..
// KW-1 leave their sums in LDS and wave 0 adds them in wave order (the same
// order on every call) to its own, which started from sc * C, and writes D.
// TRI: A lower triangular (the diagonal-block solve): the tile at r0 needs K
// up to r0 + 64 only.  CPLX: complex fp64 through the real view, with p set
// up as for gemm_lf_kernel.  K (real) is a multiple of 8.
template <int RING, int KW, bool TRI, bool CPLX>
__global__ __launch_bounds__(64 * KW) void gemm_ks_kernel(GemmParams<double> p) {
    __shared__ double red[(KW - 1) * 16 * 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c16 = lane & 15;
    const int q = lane >> 4;
    int tm, tn;
    map_tile(blockIdx.x, p.tilesM, p.tilesN, tm, tn);
    const double *__restrict__ pA = p.A;
    const double *__restrict__ pB = p.Bm;
    const int64_t lda = p.lda, ldb = p.ldb;
    // as gemm_lf_kernel: real rows 2c, 2c + 1 at k = 2q (offA0) and 2q + 1
    // (offA1), 32 rows further at +256 bytes; complex element (c, q)
    const uint32_t offA0 = CPLX ? (uint32_t)((c16 + q * lda) * 16) : (uint32_t)((2 * c16 + 2 * q * lda) * 8);
    const uint32_t offA1 = offA0 + (uint32_t)(lda * 8);
    const uint32_t offB = (uint32_t)((2 * q + c16 * ldb) * 8);
    const double sc = p.sc.re, sci = p.sc.im, gamma = p.gamma.re, gammai = p.gamma.im;
    const int64_t r0 = (int64_t)tm * 64;
    const int64_t c0 = (int64_t)tn * 16;
    // K is a multiple of 8 (the launcher's condition): whole chunks only
    const int64_t K = TRI ? (r0 + 64 < p.K ? r0 + 64 : p.K) : p.K;
    const int64_t nch = K / 8;
    const int64_t kc0 = nch * wave / KW, kfe = nch * (wave + 1) / KW;  // this wave's chunks

    d4 acc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[a] = d4{0.0, 0.0, 0.0, 0.0};
    const int64_t j = c0 + c16;
    if (wave == 0 && p.has_c && j < p.N) {  // wave 0 starts from sc * C
        const double *col = p.C + j * p.ldc;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t r = r0 + 2 * (q + 4 * v) + 32 * h;
                double x0 = 0.0, x1 = 0.0;
                if (p.c_vec && r + 1 < p.M) {
                    const d2v c2 = *reinterpret_cast<const d2v *>(col + r);
                    x0 = c2[0];
                    x1 = c2[1];
                } else {
                    if (r < p.M) x0 = col[r];
                    if (r + 1 < p.M) x1 = col[r + 1];
                }
                if constexpr (CPLX) {
                    acc[2 * h][v] = sc * x0 - sci * x1;
                    acc[2 * h + 1][v] = sc * x1 + sci * x0;
                } else {
                    acc[2 * h][v] = sc * x0;
                    acc[2 * h + 1][v] = sc * x1;
                }
            }
        }
    }

    d2v ra[RING][4], rb[RING];
    auto load = [&](int slot, int64_t kc, bool live) {
        const int64_t k0 = 8 * kc;
        const int64_t oa = r0 + k0 * lda;
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(pA + oa, live ? (p.extA - oa) * 8 : 0);
        ra[slot][0] = __builtin_bit_cast(d2v, ld16<true>(rsa, offA0));
        ra[slot][1] = __builtin_bit_cast(d2v, ld16<true>(rsa, offA0 + 256));
        if constexpr (!CPLX) {
            ra[slot][2] = __builtin_bit_cast(d2v, ld16<true>(rsa, offA1));
            ra[slot][3] = __builtin_bit_cast(d2v, ld16<true>(rsa, offA1 + 256));
        }
        const int64_t ob = k0 + c0 * ldb;
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(pB + ob, live ? (p.extB - ob) * 8 : 0);
        rb[slot] = __builtin_bit_cast(d2v, ld16<true>(rsb, offB));
    };
    auto compute = [&](const d2v (&a4)[4], const d2v &bq) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            double av[4];
            if constexpr (CPLX) {
                if (s == 0) {
                    av[0] = a4[0][0]; av[1] = a4[0][1]; av[2] = a4[1][0]; av[3] = a4[1][1];
                } else {
                    av[0] = -a4[0][1]; av[1] = a4[0][0]; av[2] = -a4[1][1]; av[3] = a4[1][0];
                }
            } else {
                av[0] = a4[2 * s][0]; av[1] = a4[2 * s][1]; av[2] = a4[2 * s + 1][0]; av[3] = a4[2 * s + 1][1];
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) acc[a] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bq[s], acc[a], 0, 0, 0);
        }
    };
#pragma unroll
    for (int u = 0; u < RING; ++u) load(u, kc0 + u, kc0 + u < kfe);
    // whole rounds, then the last chunks (as gemm_lf_kernel)
    int64_t kc = kc0;
    for (; kc + RING <= kfe; kc += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            compute(ra[u], rb[u]);
            load(u, kc + u + RING, kc + u + RING < kfe);
        }
    }
#pragma unroll
    for (int u = 0; u < RING; ++u)
        if (kc + u < kfe) compute(ra[u], rb[u]);  // uniform
    // ---- the waves' sums into wave 0, in wave order ------------------------
    if (wave > 0) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[((wave - 1) * 16 + 4 * a + v) * 64 + lane] = acc[a][v];
    }
    __syncthreads();
    if (wave != 0 || j >= p.N) return;
#pragma unroll 1
    for (int w = 1; w < KW; ++w)  // one wave's sums at a time (registers)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[a][v] += red[((w - 1) * 16 + 4 * a + v) * 64 + lane];

    // ---- D = gamma * acc, rows below `split` to D2 (as gemm_lf_kernel) ------
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t r = r0 + 2 * (q + 4 * v) + 32 * h;
            if (r >= p.M) continue;
            double x0, x1;
            if constexpr (CPLX) {
                x0 = gamma * acc[2 * h][v] - gammai * acc[2 * h + 1][v];
                x1 = gamma * acc[2 * h + 1][v] + gammai * acc[2 * h][v];
            } else {
                x0 = gamma * acc[2 * h][v];
                x1 = gamma * acc[2 * h + 1][v];
            }
            if (r + 1 < p.M && r + 1 < p.split) {
                double *dst = p.D2 + j * p.ldd2 + r;
                if (p.d2_vec) *reinterpret_cast<d2v *>(dst) = d2v{x0, x1};
                else { dst[0] = x0; dst[1] = x1; }
            } else if (r + 1 < p.M && r >= p.split) {
                double *dst = p.D + j * p.ldd + r;
                if (p.d_vec) *reinterpret_cast<d2v *>(dst) = d2v{x0, x1};
                else { dst[0] = x0; dst[1] = x1; }
            } else {
                if (r < p.split) p.D2[r + j * p.ldd2] = x0;
                else p.D[r + j * p.ldd] = x0;
                if (r + 1 < p.M) {
                    if (r + 1 < p.split) p.D2[r + 1 + j * p.ldd2] = x1;
                    else p.D[r + 1 + j * p.ldd] = x1;
                }
            }
        }
    }
}

// ---- fp32 products without LDS ---------------------------------------------
// The same structure for fp32 on v_mfma_f32_16x16x4f32 (32 cycles: twice the
// fp64 rate on half the operand bytes, so the same operand traffic per
// cycle), in chunks of 16 k:
//   * A: lane (c, q) loads rows 4c .. 4c + 3 of the wave's 64 at chunk
//     k = 4q + s (s = 0..3), 16 bytes, consecutive lanes on consecutive
//     rows; MFMA row tile a takes row 4c + a as its row c;
//   * Bm: lane (c, q) loads k = 4q .. 4q + 3 of columns c + 16b, 16 bytes;
//     k index q of MFMA step s is chunk k 4q + s on both sides;
//   * the f32 result puts MFMA row 4q + v in item v, so a lane holds output
//     rows 16q + 4v .. 16q + 4v + 3 (tiles a = 0..3): C and D move in
//     16-byte quadruples;
//   * the ragged last chunk zeroes the lanes whose k is past K, with 4-byte
//     Bm loads there.
// NBT and TRI as for gemm_lf_kernel; MINB: workgroups per CU the register
// budget is sized for.
// CPLX: complex fp32 through the real 2 x 2 embedding, p describing the real
// view as for gemm_lf_kernel (M, K, split in real rows and k; Bm, C, D, D2
// interleaved storage read as real with doubled leading dimensions; A in
// complex addressing, lda in complex elements, extA in floats).  Real rows
// 4c .. 4c+3 are complex rows 2c, 2c+1, so one 16-byte load of A(2c, k) and
// A(2c+1, k) at complex k = 2q + h feeds MFMA steps s = 2h (re, im, re, im)
// and s = 2h+1 (-im, re, -im, re): two A loads per chunk instead of four.
// The four items of a lane's output quadruple are two complex elements, so
// C is scaled by sc and the result by gamma as complex numbers.
template <int RING, int NBT, bool TRI, int MINB = 1, bool CPLX = false, int KS = 1>
__global__ __launch_bounds__(256 * KS, MINB) void gemm_lf32_kernel(GemmParams<float> p) {
    static_assert(KS == 1 || (KS == 2 && !TRI), "K split: rectangular products");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // KS = 2: eight waves, wave w on output quadrant w % 4 over half w / 4
    // of K (the halves meet through LDS, second half into the first)
    const int half = KS == 2 ? wave >> 2 : 0;
    const int qw = KS == 2 ? wave & 3 : wave;
    const int c16 = lane & 15;
    const int q = lane >> 4;
    int tm, tn;
    map_tile(blockIdx.x, p.tilesM, p.tilesN, tm, tn);
    const float *__restrict__ pA = p.A;
    const float *__restrict__ pB = p.Bm;
    const int64_t lda = p.lda, ldb = p.ldb;
    uint32_t offA[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if constexpr (CPLX) offA[s] = (uint32_t)((2 * c16 + (2 * q + (s & 1)) * lda) * 8);  // s < 2 used
        else offA[s] = (uint32_t)((4 * c16 + (4 * q + s) * lda) * 4);
    }
    uint32_t offB[NBT];
#pragma unroll
    for (int b = 0; b < NBT; ++b) offB[b] = (uint32_t)((4 * q + (c16 + 16 * (int64_t)b) * ldb) * 4);
    const float sc = (float)p.sc.re, gamma = (float)p.gamma.re;
    const float sci = (float)p.sc.im, gammai = (float)p.gamma.im;  // complex only

    auto run_tile = [&](const int64_t r0, const int64_t c0, const int64_t kb, const int64_t K) {
        f4 acc[4][NBT];
#pragma unroll
        for (int b = 0; b < NBT; ++b) {
            const int64_t j = c0 + c16 + 16 * b;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t r = r0 + 16 * q + 4 * v;
                float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (p.has_c && j < p.N && half == 0) {
                    const float *col = p.C + j * p.ldc;
                    if (p.c_vec && r + 3 < p.M) {
                        const f4 c4 = *reinterpret_cast<const f4 *>(col + r);
                        x[0] = c4[0]; x[1] = c4[1]; x[2] = c4[2]; x[3] = c4[3];
                    } else {
#pragma unroll
                        for (int a = 0; a < 4; ++a)
                            if (r + a < p.M) x[a] = col[r + a];
                    }
                }
                if constexpr (CPLX) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {  // complex sc * C
                        acc[2 * h][b][v] = sc * x[2 * h] - sci * x[2 * h + 1];
                        acc[2 * h + 1][b][v] = sc * x[2 * h + 1] + sci * x[2 * h];
                    }
                } else {
#pragma unroll
                    for (int a = 0; a < 4; ++a) acc[a][b][v] = sc * x[a];
                }
            }
        }

        f4 ra[RING][4], rb[RING][NBT];
        auto load = [&](int slot, int64_t k0, bool live) {
            const int64_t oa = r0 + k0 * lda;
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(pA + oa, live ? (p.extA - oa) * 4 : 0);
            if constexpr (CPLX) {
                ra[slot][0] = __builtin_bit_cast(f4, ld16<true>(rsa, offA[0]));
                ra[slot][1] = __builtin_bit_cast(f4, ld16<true>(rsa, offA[1]));
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) ra[slot][s] = __builtin_bit_cast(f4, ld16<true>(rsa, offA[s]));
            }
            const int64_t ob = k0 + c0 * ldb;
            const __amdgpu_buffer_rsrc_t rsb = make_rsrc(pB + ob, live ? (p.extB - ob) * 4 : 0);
#pragma unroll
            for (int b = 0; b < NBT; ++b) rb[slot][b] = __builtin_bit_cast(f4, ld16<true>(rsb, offB[b]));
        };
        auto compute = [&](const f4 (&a4)[4], const f4 (&bq)[NBT]) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                f4 av;
                if constexpr (CPLX) {
                    const f4 x = a4[s >> 1];
                    if (s & 1) av = f4{-x[1], x[0], -x[3], x[2]};
                    else av = x;
                } else {
                    av = a4[s];
                }
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < NBT; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bq[b][s], acc[a][b], 0, 0, 0);
            }
        };
        const int64_t nkf = (K - kb) / 16;  // full chunks
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            load(u, kb + 16 * u, u < nkf);
            if constexpr (CPLX) __builtin_amdgcn_sched_barrier(0);
        }
        // whole rounds, then the last chunks (as gemm_lf_kernel)
        int64_t kc = 0;
        for (; kc + RING <= nkf; kc += RING) {
#pragma unroll
            for (int u = 0; u < RING; ++u) {
                compute(ra[u], rb[u]);
                load(u, kb + 16 * (kc + u + RING), kc + u + RING < nkf);
                // complex: keep each slot's loads with their slot, which holds
                // every wait of the ring at its full depth (complex fp32
                // 8192^2 16.5 -> 16.1 ms); for real data the free schedule
                // was faster even with shallower waits
                if constexpr (CPLX) __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int u = 0; u < RING; ++u)
            if (kc + u < nkf) compute(ra[u], rb[u]);  // uniform
        const int kr = (int)(K - kb - 16 * nkf);
        if (kr > 0) {
            const int64_t k0 = kb + 16 * nkf;
            const int64_t oa = r0 + k0 * lda;
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(pA + oa, (p.extA - oa) * 4);
            const uint32_t dead = 0xfffffff0u;
            f4 ta[4], tb[NBT];
            if constexpr (CPLX) {
                // the real K is even: a complex k is whole or absent
                ta[0] = __builtin_bit_cast(f4, ld16<true>(rsa, 4 * q < kr ? offA[0] : dead));
                ta[1] = __builtin_bit_cast(f4, ld16<true>(rsa, 4 * q + 2 < kr ? offA[1] : dead));
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    ta[s] = __builtin_bit_cast(f4, ld16<true>(rsa, 4 * q + s < kr ? offA[s] : dead));
            }
            const int64_t ob = k0 + c0 * ldb;
            const __amdgpu_buffer_rsrc_t rsb = make_rsrc(pB + ob, (p.extB - ob) * 4);
#pragma unroll
            for (int b = 0; b < NBT; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    tb[b][s] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(rsb, 4 * q + s < kr ? offB[b] + 4 * s : dead, 0, 0));
            compute(ta, tb);
        }

        if constexpr (KS == 2) {
            // the second half's sums join the first's through LDS
            __shared__ f4 red[4][4][NBT][64];
            if (half == 1) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < NBT; ++b) red[qw][a][b][lane] = acc[a][b];
            }
            __syncthreads();
            if (half == 1) return;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < NBT; ++b) acc[a][b] += red[qw][a][b][lane];
        }

#pragma unroll
        for (int b = 0; b < NBT; ++b) {
            const int64_t j = c0 + c16 + 16 * b;
            if (j >= p.N) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t r = r0 + 16 * q + 4 * v;
                if (r >= p.M) continue;
                float out[4];
                if constexpr (CPLX) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {  // complex gamma * acc
                        out[2 * h] = gamma * acc[2 * h][b][v] - gammai * acc[2 * h + 1][b][v];
                        out[2 * h + 1] = gamma * acc[2 * h + 1][b][v] + gammai * acc[2 * h][b][v];
                    }
                } else {
#pragma unroll
                    for (int a = 0; a < 4; ++a) out[a] = gamma * acc[a][b][v];
                }
                if (r + 3 < p.M && r + 3 < p.split) {
                    float *dst = p.D2 + j * p.ldd2 + r;
                    if (p.d2_vec) *reinterpret_cast<f4 *>(dst) = f4{out[0], out[1], out[2], out[3]};
                    else for (int a = 0; a < 4; ++a) dst[a] = out[a];
                } else if (r + 3 < p.M && r >= p.split) {
                    float *dst = p.D + j * p.ldd + r;
                    if (p.d_vec) *reinterpret_cast<f4 *>(dst) = f4{out[0], out[1], out[2], out[3]};
                    else for (int a = 0; a < 4; ++a) dst[a] = out[a];
                } else {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int64_t ii = r + a;
                        if (ii >= p.M) break;
                        if (ii < p.split) p.D2[ii + j * p.ldd2] = out[a];
                        else p.D[ii + j * p.ldd] = out[a];
                    }
                }
            }
        }
    };

    if constexpr (TRI) {
        const int T = (int)((p.M + 63) / 64);
        const int64_t c0 = (int64_t)tn * 64 * NBT + (int64_t)wave * 16 * NBT;
        const int t1 = T - 1 - tm;
        for (int pass = 0; pass < (t1 != tm ? 2 : 1); ++pass) {
            const int64_t r0 = (int64_t)(pass == 0 ? tm : t1) * 64;
            run_tile(r0, c0, 0, r0 + 64 < p.K ? r0 + 64 : p.K);
        }
    } else {
        const int64_t r0 = (int64_t)tm * 128 + (qw & 1) * 64;
        const int64_t c0 = (int64_t)tn * 32 * NBT + (int64_t)(qw >> 1) * 16 * NBT;
        if constexpr (KS == 2) {
            // halves split at a chunk boundary; the second takes the ragged end
            const int64_t kmid = 16 * (((p.K + 15) / 16) / 2);
            run_tile(r0, c0, half ? kmid : 0, half ? p.K : kmid);
        } else {
            run_tile(r0, c0, 0, p.K);
        }
    }
}

inline bool aligned16(const void *ptr, int64_t ld, size_t es) {
    return (reinterpret_cast<uintptr_t>(ptr) % 16) == 0 && ((int64_t)es * ld) % 16 == 0;
}

// Kernel parameters and grid of descriptor g on an MT x NT tile.  Returns
// hipSuccess with grid.x == 0 when there is nothing to compute.
template <typename T, int MT, int NT>
hipError_t tile_params(const GemmDesc &g, GemmParams<T> &p, dim3 &grid) {
    constexpr bool CPLX = GemmTraits<T>::kCplx;
    grid = dim3(0u, 1u, 1u);
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
    p.gamma = g.gamma;
    p.has_c = (g.C != nullptr) && (g.beta.re != 0.0 || g.beta.im != 0.0);
    if (g.gamma.re == 0.0 && g.gamma.im == 0.0) {
        // D = beta * C: no product at all
        p.K = 0;
        p.gamma = Scalar{1.0, 0.0};
        p.sc = g.beta;
    } else if (CPLX) {
        // sc = beta / gamma (complex), exact when gamma = +-1
        const double den = g.gamma.re * g.gamma.re + g.gamma.im * g.gamma.im;
        if (g.gamma.im == 0.0)
            p.sc = Scalar{g.beta.re / g.gamma.re, g.beta.im / g.gamma.re};
        else
            p.sc = Scalar{(g.beta.re * g.gamma.re + g.beta.im * g.gamma.im) / den,
                          (g.beta.im * g.gamma.re - g.beta.re * g.gamma.im) / den};
    } else {
        p.sc = Scalar{g.beta.re / g.gamma.re, 0.0};
    }
    p.extA = p.K > 0 ? (p.K - 1) * p.lda + p.M : 0;
    p.extB = p.K > 0 ? (p.N - 1) * p.ldb + p.K : 0;
    const size_t es = sizeof(T);
    p.a_vec = aligned16(g.A, g.lda, es);
    p.b_vec = aligned16(g.Bm, g.ldb, es);
    p.c_vec = p.has_c ? aligned16(g.C, g.ldc, es) : 0;
    p.d_vec = aligned16(g.D, g.ldd, es);
    p.d2_vec = aligned16(p.D2, p.ldd2, es);
    const int64_t Mr = CPLX ? 2 * g.M : g.M;
    const int64_t tM = (Mr + MT - 1) / MT;
    const int64_t tN = (g.N + NT - 1) / NT;
    if (tM <= 0 || tN <= 0) return hipSuccess;
    if (tM * tN > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    p.tilesM = (int)tM;
    p.tilesN = (int)tN;
    const int64_t nz = g.batch > 1 ? g.batch : 1;
    if (nz > 65535) return hipErrorInvalidConfiguration;
    p.binner = nz > 1 ? (int)g.binner : 1;
    p.sAo = g.sAo; p.sAi = g.sAi; p.sBo = g.sBo; p.sBi = g.sBi;
    p.sCo = g.sCo; p.sCi = g.sCi; p.sDo = g.sDo; p.sDi = g.sDi;
    p.sKo = nz > 1 && g.a_lower ? g.sKo : 0;
    p.fold = g.a_lower && p.sKo == 0;
    if (nz > 1) {
        if (g.split != 0 || g.binner < 1) return hipErrorInvalidValue;
        // every problem's operands keep the alignment of the first
        const auto al = [&](int64_t o, int64_t i) { return (o * (int64_t)es) % 16 == 0 && (i * (int64_t)es) % 16 == 0; };
        if (!al(g.sAo, g.sAi)) p.a_vec = 0;
        if (!al(g.sBo, g.sBi)) p.b_vec = 0;
        if (!al(g.sCo, g.sCi)) p.c_vec = 0;
        if (!al(g.sDo, g.sDi)) p.d_vec = p.d2_vec = 0;
    }
    const int64_t rowsM = p.fold ? (tM + 1) / 2 : tM;  // folded triangle: pairs of row tiles
    grid = dim3((unsigned)(rowsM * tN), (unsigned)nz);
    return hipSuccess;
}

template <typename T, int MT, int NT, int KT>
hipError_t launch_tile(const GemmDesc &g, hipStream_t st) {
    GemmParams<T> p;
    dim3 grid;
    hipError_t e = tile_params<T, MT, NT>(g, p, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    const bool vec = p.a_vec && p.b_vec;
    if (g.b_lower) {
        // the shapes launched with it (the inversion's second product)
        if constexpr ((MT == 64 && NT == 32) || (MT == 32 && NT == 32) || (MT == 64 && NT == 64)) {
            if (vec) hipLaunchKernelGGL((gemm_kernel<T, MT, NT, KT, false, true, true>), grid, dim3(256), 0, st, p);
            else hipLaunchKernelGGL((gemm_kernel<T, MT, NT, KT, false, false, true>), grid, dim3(256), 0, st, p);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (g.a_lower) {
        if (vec) hipLaunchKernelGGL((gemm_kernel<T, MT, NT, KT, true, true>), grid, dim3(256), 0, st, p);
        else hipLaunchKernelGGL((gemm_kernel<T, MT, NT, KT, true, false>), grid, dim3(256), 0, st, p);
    } else {
        if (vec) hipLaunchKernelGGL((gemm_kernel<T, MT, NT, KT, false, true>), grid, dim3(256), 0, st, p);
        else hipLaunchKernelGGL((gemm_kernel<T, MT, NT, KT, false, false>), grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

// Operands whose leading dimension is too large for 32-bit buffer offsets
// inside a tile: the 64 x 32 tile with 64-bit global loads (WIDE).
template <typename T, int KT>
hipError_t launch_wide(const GemmDesc &g, hipStream_t st) {
    GemmParams<T> p;
    dim3 grid;
    hipError_t e = tile_params<T, 64, 32>(g, p, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    if (g.b_lower)
        hipLaunchKernelGGL((gemm_kernel<T, 64, 32, KT, false, false, true, true>), grid, dim3(256), 0, st, p);
    else if (g.a_lower)
        hipLaunchKernelGGL((gemm_kernel<T, 64, 32, KT, true, false, false, true>), grid, dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((gemm_kernel<T, 64, 32, KT, false, false, false, true>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// fp64 single products on gemm_lf_kernel (TRSM_GEMM_LF=0 turns it off for
// tuning and tests).
bool use_gemm_lf() {
    const char *e = std::getenv("TRSM_GEMM_LF");
    return !(e && e[0] == '0');
}

hipError_t launch_lf(const GemmDesc &g, hipStream_t st) {
    GemmParams<double> p;
    dim3 grid;
    hipError_t e = tile_params<double, 128, 128>(g, p, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    hipLaunchKernelGGL((gemm_lf_kernel<3, 4, false>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// The diagonal inversion's batched fp64 products on gemm_lf_kernel, 64 x 16
// per wave: the triangular first product folds row tiles (four waves side by
// side on 64 columns), the second (triangular Bm) runs 128 x 32 workgroups
// whose waves start K at their first column.  Taken from 256 workgroups
// (TRSM_INV_LF_MIN overrides; TRSM_INV_LF=0 keeps the LDS tile): with fewer,
// one wave per SIMD at most cannot hide its loads.  Measured (whole solves,
// three rounds on one box): fp64 8192 x 64 0.419 -> 0.411 ms, 8192 x 256
// 0.599 -> 0.593 ms, 4096^2 and 8192^2 unchanged within noise; taken for
// every level it lost (4096^2 inversion 133 -> 145 us).
bool use_inv_lf(const GemmDesc &g, size_t es) {
    const char *e = std::getenv("TRSM_INV_LF");
    if ((e && e[0] == '0') || !use_gemm_lf() || g.split != 0 || g.D2 != nullptr) return false;
    const auto al = [&](int64_t o, int64_t i) { return (o * (int64_t)es) % 16 == 0 && (i * (int64_t)es) % 16 == 0; };
    if (!(aligned16(g.A, g.lda, es) && aligned16(g.Bm, g.ldb, es) && al(g.sAo, g.sAi) && al(g.sBo, g.sBi)))
        return false;
    const int64_t Mr = es == 16 ? 2 * g.M : g.M;  // real rows (complex: the real view)
    const int64_t wg = g.batch * (g.a_lower ? (((Mr + 63) / 64 + 1) / 2) * ((g.N + 63) / 64)
                                            : ((Mr + 127) / 128) * ((g.N + 31) / 32));
    const char *m = std::getenv("TRSM_INV_LF_MIN");
    return wg >= (m ? std::atoll(m) : 256);
}

template <int RING>
hipError_t launch_lf_batched(const GemmDesc &g, hipStream_t st) {
    GemmParams<double> p;
    dim3 grid;
    hipError_t e = tile_params<double, 128, 128>(g, p, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    if (g.a_lower) {
        p.tilesM = (int)(((g.M + 63) / 64 + 1) / 2);  // row-tile pairs
        p.tilesN = (int)((g.N + 63) / 64);
        grid = dim3((unsigned)(p.tilesM * p.tilesN), grid.y);
        hipLaunchKernelGGL((gemm_lf_kernel<RING, 1, true, false, true, false>), grid, dim3(256), 0, st, p);
    } else {
        p.tilesM = (int)((g.M + 127) / 128);
        p.tilesN = (int)((g.N + 31) / 32);
        if (g.b_lower) p.tilesN = (p.tilesN + 1) / 2;  // folded column blocks
        grid = dim3((unsigned)(p.tilesM * p.tilesN), grid.y);
        if (g.b_lower)
            hipLaunchKernelGGL((gemm_lf_kernel<RING, 1, false, false, true, true>), grid, dim3(256), 0, st, p);
        else
            hipLaunchKernelGGL((gemm_lf_kernel<RING, 1, false, false, true, false>), grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

// fp64 updates on 128 x 32 NBT workgroups of gemm_lf_kernel (64 x 16 NBT per
// wave), sized for two workgroups per CU.
template <int RING, int NBT>
hipError_t launch_lf_n(const GemmDesc &g, hipStream_t st) {
    GemmParams<double> p;
    dim3 grid;
    hipError_t e = tile_params<double, 128, 128>(g, p, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    p.tilesM = (int)((g.M + 127) / 128);
    p.tilesN = (int)((g.N + 32 * NBT - 1) / (32 * NBT));
    grid = dim3((unsigned)(p.tilesM * p.tilesN), 1u);
    hipLaunchKernelGGL((gemm_lf_kernel<RING, NBT, false>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// Updates with 256 to 511 tiles of 128 x 128 in rounds of 256 more than 3/4
// full, on 128 x 64 workgroups (64 x 32 per wave, two per CU, as fp32 does)
// instead of the LDS tiles (TRSM_LF_MID=0 turns this off for tuning).
// Measured (whole solves, three rounds on one box): fp64 4096^2 1.326 ->
// 1.233 ms, 8192 x 2048 2.723 -> 2.709; complex 8192 x 2048 8.46-8.48 ->
// 8.44, 8192 x 1024 5.040 -> 5.008, 2048^2 0.847 -> 0.832 ms.
bool use_lf_mid(int64_t t128) {
    const char *e = std::getenv("TRSM_LF_MID");
    return !(e && e[0] == '0') && t128 >= 256 && t128 < 512 && 4 * t128 > 3 * 256 * ((t128 + 255) / 256);
}

// The real view of a complex fp64 product for the LDS-free kernels: M and
// K doubled (real rows and k), Bm, C, D and D2 read as interleaved real with
// doubled leading dimensions, A kept in complex addressing (lda in complex
// elements, extA in doubles).
GemmParams<double> real_view(const GemmParams<cplx> &pc) {
    GemmParams<double> p{};
    p.M = 2 * pc.M;
    p.N = pc.N;
    p.K = 2 * pc.K;
    p.A = reinterpret_cast<const double *>(pc.A);
    p.lda = pc.lda;
    p.extA = 2 * pc.extA;
    p.Bm = reinterpret_cast<const double *>(pc.Bm);
    p.ldb = 2 * pc.ldb;
    p.extB = 2 * pc.extB;
    p.C = reinterpret_cast<const double *>(pc.C);
    p.ldc = 2 * pc.ldc;
    p.D = reinterpret_cast<double *>(pc.D);
    p.ldd = 2 * pc.ldd;
    p.D2 = reinterpret_cast<double *>(pc.D2);
    p.ldd2 = 2 * pc.ldd2;
    p.split = 2 * pc.split;
    p.sc = pc.sc;
    p.gamma = pc.gamma;
    p.has_c = pc.has_c;
    p.a_vec = pc.a_vec;
    p.b_vec = pc.b_vec;
    p.c_vec = pc.c_vec;
    p.d_vec = pc.d_vec;
    p.d2_vec = pc.d2_vec;
    p.binner = 1;
    return p;
}

// Complex fp64 single products on gemm_lf_kernel through the real view.
hipError_t launch_lf_cplx(const GemmDesc &g, hipStream_t st) {
    GemmParams<cplx> pc;
    dim3 grid;
    hipError_t e = tile_params<cplx, 128, 128>(g, pc, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    GemmParams<double> p = real_view(pc);
    p.tilesM = (int)((p.M + 127) / 128);
    p.tilesN = (int)((p.N + 127) / 128);
    grid = dim3((unsigned)(p.tilesM * p.tilesN), 1u);
    hipLaunchKernelGGL((gemm_lf_kernel<3, 4, false, true>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// The inversion's batched complex fp64 products on gemm_lf_kernel through
// the real view (as launch_lf_batched; batch strides in doubles).
template <int RING>
hipError_t launch_lf_batched_cplx(const GemmDesc &g, hipStream_t st) {
    GemmParams<cplx> pc;
    dim3 grid;
    hipError_t e = tile_params<cplx, 128, 128>(g, pc, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    GemmParams<double> p = real_view(pc);
    p.binner = pc.binner;
    p.sAo = 2 * pc.sAo; p.sAi = 2 * pc.sAi; p.sBo = 2 * pc.sBo; p.sBi = 2 * pc.sBi;
    p.sCo = 2 * pc.sCo; p.sCi = 2 * pc.sCi; p.sDo = 2 * pc.sDo; p.sDi = 2 * pc.sDi;
    if (g.a_lower) {
        p.tilesM = (int)(((p.M + 63) / 64 + 1) / 2);  // real row-tile pairs
        p.tilesN = (int)((p.N + 63) / 64);
        grid = dim3((unsigned)(p.tilesM * p.tilesN), grid.y);
        hipLaunchKernelGGL((gemm_lf_kernel<RING, 1, true, true, true, false>), grid, dim3(256), 0, st, p);
    } else {
        p.tilesM = (int)((p.M + 127) / 128);
        p.tilesN = (int)((p.N + 31) / 32);
        if (g.b_lower) p.tilesN = (p.tilesN + 1) / 2;  // folded column blocks
        grid = dim3((unsigned)(p.tilesM * p.tilesN), grid.y);
        if (g.b_lower)
            hipLaunchKernelGGL((gemm_lf_kernel<RING, 1, false, true, true, true>), grid, dim3(256), 0, st, p);
        else
            hipLaunchKernelGGL((gemm_lf_kernel<RING, 1, false, true, true, false>), grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

// Updates with 64 to 255 such tiles: 128 x 32 workgroups (64 x 16 per wave,
// a ring of four), four times the workgroups.  TRSM_LF_LOW sets the lower
// bound (0: off).  Measured (whole solves, three rounds on one box, against
// the 64 x 32 and 64 x 64 LDS tiles): fp64 2048^2 0.301 -> 0.287 ms,
// 8192 x 1024 1.565 -> 1.524; complex 2048^2 0.808 -> 0.790, 8192 x 512
// 2.86 -> 2.82 ms.
bool use_lf_low(int64_t t128) {
    const char *e = std::getenv("TRSM_LF_LOW");
    const int64_t lo = e ? std::atoll(e) : 64;
    return lo > 0 && t128 >= lo && t128 < 256;
}

// Complex fp64 updates through the real view on 128 x 32 NBT workgroups.
template <int RING, int NBT>
hipError_t launch_lf_cplx_n(const GemmDesc &g, hipStream_t st) {
    GemmParams<cplx> pc;
    dim3 grid;
    hipError_t e = tile_params<cplx, 128, 128>(g, pc, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    GemmParams<double> p = real_view(pc);
    p.tilesM = (int)((p.M + 127) / 128);
    p.tilesN = (int)((p.N + 32 * NBT - 1) / (32 * NBT));
    grid = dim3((unsigned)(p.tilesM * p.tilesN), 1u);
    hipLaunchKernelGGL((gemm_lf_kernel<RING, NBT, false, true>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// Complex fp64 triangular solve products on gemm_lf_kernel through the real
// view: folded pairs of 64-row real tiles, 16 NBT columns per wave.
template <int RING, int NBT>
hipError_t launch_lf_tri_cplx(const GemmDesc &g, hipStream_t st) {
    GemmParams<cplx> pc;
    dim3 grid;
    hipError_t e = tile_params<cplx, 128, 128>(g, pc, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    GemmParams<double> p = real_view(pc);
    p.tilesM = (int)(((p.M + 63) / 64 + 1) / 2);
    p.tilesN = (int)((p.N + 64 * NBT - 1) / (64 * NBT));
    grid = dim3((unsigned)(p.tilesM * p.tilesN), 1u);
    hipLaunchKernelGGL((gemm_lf_kernel<RING, NBT, true, true>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// fp64 and complex fp64 products that split-K would cut, on gemm_ks_kernel:
// 64 x 16 tiles, KW = the split-K factor (at most 8) waves on each.
template <int KW>
hipError_t launch_ks_kw(const GemmParams<double> &p, bool tri, bool cplx_view, hipStream_t st) {
    const dim3 grid((unsigned)(p.tilesM * p.tilesN), 1u);
    const dim3 block(64 * KW);
    if (tri && cplx_view) hipLaunchKernelGGL((gemm_ks_kernel<3, KW, true, true>), grid, block, 0, st, p);
    else if (tri) hipLaunchKernelGGL((gemm_ks_kernel<3, KW, true, false>), grid, block, 0, st, p);
    else if (cplx_view) hipLaunchKernelGGL((gemm_ks_kernel<3, KW, false, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((gemm_ks_kernel<3, KW, false, false>), grid, block, 0, st, p);
    return hipGetLastError();
}

hipError_t launch_ks(int dtype, const GemmDesc &g, int parts, hipStream_t st) {
    GemmParams<double> p;
    dim3 grid;
    hipError_t e;
    if (dtype == C64F) {
        GemmParams<cplx> pc;
        e = tile_params<cplx, 64, 16>(g, pc, grid);
        if (e != hipSuccess || grid.x == 0) return e;
        p = real_view(pc);
    } else {
        e = tile_params<double, 64, 16>(g, p, grid);
        if (e != hipSuccess || grid.x == 0) return e;
    }
    const int64_t tM = (p.M + 63) / 64, tN = (p.N + 15) / 16;
    if (tM * tN > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    p.tilesM = (int)tM;
    p.tilesN = (int)tN;
    const bool tri = g.a_lower != 0, cv = dtype == C64F;
    if (parts >= 8) return launch_ks_kw<8>(p, tri, cv, st);
    if (parts >= 4) return launch_ks_kw<4>(p, tri, cv, st);
    return launch_ks_kw<2>(p, tri, cv, st);
}

// Whether a split-K product runs on gemm_ks_kernel: fp64 or complex fp64, a
// single product with K a multiple of 8 (split K is always a multiple of
// 256) and 16-byte aligned A and Bm whose tiles stay within 32-bit buffer
// offsets (as gemm_launch's non-wide path), with at least 256 output tiles
// of 64 x 16 real rows x columns: with fewer the workgroups are too few to
// hide their latency, and the batched partial products measured faster
// (fp64 8192 x 64, IB 1024: 0.418 ms against 0.441; 8192 x 256: 0.697
// against 0.618 in favour of this form).  TRSM_GEMM_KS=0 keeps the batched
// partial products, =1 takes this form whatever the tile count (tuning and
// tests).
bool use_ks(int dtype, const GemmDesc &g) {
    if (dtype != R64F && dtype != C64F) return false;
    const char *e = std::getenv("TRSM_GEMM_KS");
    if ((e && e[0] == '0') || !use_gemm_lf()) return false;
    const int64_t Mr = dtype == C64F ? 2 * g.M : g.M;
    if (!(e && e[0] == '1') && ((Mr + 63) / 64) * ((g.N + 15) / 16) < 256) return false;
    const int64_t es = (int64_t)dtype_size(dtype);
    if (g.batch > 1 || g.b_lower || g.M <= 0 || g.N <= 0 || g.K % 8 != 0) return false;
    if (g.lda > (0x7fffffffLL - 4096) / (es * 32) || g.ldb > (0x7fffffffLL - 4096) / (es * 128)) return false;
    return aligned16(g.A, g.lda, es) && aligned16(g.Bm, g.ldb, es);
}

// Triangular fp64 product (the diagonal-block solve): workgroups of four
// 64 x 32 waves over 128 columns, each wave on the row-tile pair (i, T-1-i),
// with a ring of five chunks.  Measured on the 1024 x 8192 solve of fp64
// 8192^2: 168 us with the 64 x 32 wave tile and a ring of 3, 162 with 4,
// 158 with 5; a 64 x 64 wave tile (one wave per SIMD) 178 us; the LDS tile
// (64 x 128) 171 us.
template <int RING = 5, int NBT = 2>
hipError_t launch_lf_tri(const GemmDesc &g, hipStream_t st) {
    GemmParams<double> p;
    dim3 grid;
    hipError_t e = tile_params<double, 64, 128>(g, p, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    const int64_t T = (g.M + 63) / 64;
    p.tilesM = (int)((T + 1) / 2);  // row-tile pairs
    p.tilesN = (int)((g.N + 64 * NBT - 1) / (64 * NBT));
    grid = dim3((unsigned)(p.tilesM * p.tilesN), 1u);
    hipLaunchKernelGGL((gemm_lf_kernel<RING, NBT, true>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// fp32 single products on gemm_lf32_kernel: the update tile 128 x 128
// (64 x 64 per wave), the triangular product's wave tile 64 x 32.
template <int RING, int NBT, bool TRI, int MINB = 1, int KS = 1>
hipError_t launch_lf32(const GemmDesc &g, hipStream_t st) {
    GemmParams<float> p;
    dim3 grid;
    hipError_t e = tile_params<float, 128, 128>(g, p, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    if (TRI) {
        p.tilesM = (int)(((g.M + 63) / 64 + 1) / 2);
        p.tilesN = (int)((g.N + 64 * NBT - 1) / (64 * NBT));
    } else {
        p.tilesM = (int)((g.M + 127) / 128);
        p.tilesN = (int)((g.N + 32 * NBT - 1) / (32 * NBT));
    }
    grid = dim3((unsigned)(p.tilesM * p.tilesN), 1u);
    hipLaunchKernelGGL((gemm_lf32_kernel<RING, NBT, TRI, MINB, false, KS>), grid, dim3(256 * KS), 0, st, p);
    return hipGetLastError();
}

// Complex fp32 products on gemm_lf32_kernel through the real view (as
// real_view for complex fp64: M, K and split doubled, Bm, C, D, D2 read as
// interleaved floats with doubled leading dimensions, A in complex
// addressing with extA in floats).
template <int RING, int NBT, bool TRI, int MINB = 1>
hipError_t launch_lf32_cplx(const GemmDesc &g, hipStream_t st) {
    GemmParams<cplx32> pc;
    dim3 grid;
    hipError_t e = tile_params<cplx32, 128, 128>(g, pc, grid);
    if (e != hipSuccess || grid.x == 0) return e;
    if (grid.y > 1) return hipErrorInvalidValue;
    GemmParams<float> p{};
    p.M = 2 * pc.M;
    p.N = pc.N;
    p.K = 2 * pc.K;
    p.A = reinterpret_cast<const float *>(pc.A);
    p.lda = pc.lda;
    p.extA = 2 * pc.extA;
    p.Bm = reinterpret_cast<const float *>(pc.Bm);
    p.ldb = 2 * pc.ldb;
    p.extB = 2 * pc.extB;
    p.C = reinterpret_cast<const float *>(pc.C);
    p.ldc = 2 * pc.ldc;
    p.D = reinterpret_cast<float *>(pc.D);
    p.ldd = 2 * pc.ldd;
    p.D2 = reinterpret_cast<float *>(pc.D2);
    p.ldd2 = 2 * pc.ldd2;
    p.split = 2 * pc.split;
    p.sc = pc.sc;
    p.gamma = pc.gamma;
    p.has_c = pc.has_c;
    p.a_vec = pc.a_vec;
    p.b_vec = pc.b_vec;
    p.c_vec = pc.c_vec;
    p.d_vec = pc.d_vec;
    p.d2_vec = pc.d2_vec;
    p.binner = 1;
    if (TRI) {
        p.tilesM = (int)(((p.M + 63) / 64 + 1) / 2);
        p.tilesN = (int)((p.N + 64 * NBT - 1) / (64 * NBT));
    } else {
        p.tilesM = (int)((p.M + 127) / 128);
        p.tilesN = (int)((p.N + 32 * NBT - 1) / (32 * NBT));
    }
    grid = dim3((unsigned)(p.tilesM * p.tilesN), 1u);
    hipLaunchKernelGGL((gemm_lf32_kernel<RING, NBT, TRI, MINB, true>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

// The LDS-free fp32 forms for complex fp32, by the fp32 rules on the real
// view; TRSM_LF_C32=0 keeps the LDS tiles.
hipError_t launch_c32_lf(const GemmDesc &g, hipStream_t st, bool &taken) {
    taken = false;
    const char *e = std::getenv("TRSM_LF_C32");
    if ((e && e[0] == '0') || !use_gemm_lf() || g.batch > 1 || g.b_lower || !aligned16(g.A, g.lda, 8) ||
        !aligned16(g.Bm, g.ldb, 8))
        return hipSuccess;
    const int64_t Mr = 2 * g.M;
    const int64_t tN128 = (g.N + 127) / 128;
    taken = true;
    if (g.a_lower) {
        const int64_t p128 = ((Mr + 63) / 64 + 1) / 2 * tN128;
        if (p128 >= 512) return launch_lf32_cplx<5, 2, true>(g, st);
        if (p128 >= 256 && 4 * p128 > 3 * 256 * ((p128 + 255) / 256)) return launch_lf32_cplx<3, 1, true, 2>(g, st);
        if (p128 >= 64 && p128 < 256) return launch_lf32_cplx<3, 1, true, 2>(g, st);
    } else if (Mr > 64) {
        const int64_t t128 = ((Mr + 127) / 128) * tN128;
        if (t128 >= 512 && 4 * t128 >= 3 * 512 * ((t128 + 511) / 512)) return launch_lf32_cplx<5, 4, false>(g, st);
        if (t128 >= 256 && t128 < 512 && 4 * t128 > 3 * 256 * ((t128 + 255) / 256))
            return launch_lf32_cplx<3, 2, false, 2>(g, st);
        if (t128 >= 64 && t128 < 256) return launch_lf32_cplx<4, 1, false, 2>(g, st);
    }
    taken = false;
    return hipSuccess;
}

// Kernel and tile, from timings on MI355X of whole blocked solves.  Aligned
// single products with enough tiles go to the LDS-free kernels first (the
// rules in the branches below, with their measurements); what remains takes
// an LDS tile of gemm_kernel:
//   * 64 x 32 for the triangular solve products (each workgroup folds two
//     row tiles, so twice as many column tiles keep the CUs busy; wider
//     tiles for large fp64 and complex ones, see below), for
//     updates too small to give 1024 tiles of 64 x 64, and for split-K
//     chunks; the diagonal inversion's batched products as below;
//   * 128 x 64 (fp64) or 64 x 128 (complex, whose 64 real rows are 32
//     complex rows) for updates that give at least 2048 such tiles: at three
//     of these workgroups per CU, fewer leave a last round that runs the
//     chip part empty;
//   * 64 x 64 otherwise;
//   * for fp64, 128 x 128 ahead of all of these once it gives at least 512
//     tiles in rounds of 512 at least 3/4 full (two per CU, which is all its
//     254 VGPRs and 70 KB of LDS allow, so the first round fills the chip).  Each wave then holds 64 x 64
//     results, which halves the operand traffic per product against 64 x 64
//     tiles.  Measured on the left-looking updates of fp64 8192^2 (M = 1024,
//     N = 8192): 61.3 -> 63.4 TFLOP/s at K = 7168, the solve 9.50 -> 9.27 ms.
//     For fp32 and complex data it lost or spills.  (Aligned fp64 products
//     of that size now run the LDS-free 128 x 128 form instead.)
template <typename T, int KT>
hipError_t launch_sized(const GemmDesc &g, hipStream_t st) {
    // The batched triangular products of the diagonal inversion (split-K
    // chunks have sKo > 0): 32 x 32 tiles for fp32, twice the workgroups of
    // 64 x 32 for its few large pairs (fp32 4096^2: inversion 93 -> 87 us),
    // 64 x 64 for complex fp64 (complex 8192 x 2048: 457 -> 421 us).  The
    // tile changes no element's order of operations: the inverses are
    // bitwise the same.
    if (g.batch > 1 && (g.b_lower || (g.a_lower && g.sKo == 0))) {
        if constexpr (std::is_same<T, float>::value) return launch_tile<T, 32, 32, KT>(g, st);
        if constexpr (std::is_same<T, cplx>::value) {
            if (use_inv_lf(g, 16)) return launch_lf_batched_cplx<4>(g, st);
            return launch_tile<T, 64, 64, KT>(g, st);
        }
        if constexpr (std::is_same<T, double>::value) {
            if (use_inv_lf(g, 8)) return launch_lf_batched<4>(g, st);
        }
    }
    // fp32 single products with 64 or more 128-wide tiles run without LDS
    // (first measured on fp32 8192^2: the solve 4.56 -> 4.30 ms, updates 6 %
    // and triangular products 7 % faster than the LDS tiles; the smaller
    // shapes followed once each had a form sized for them, below)
    if constexpr (std::is_same<T, float>::value) {
        if (g.batch <= 1 && !g.b_lower) {
            const bool lf = use_gemm_lf() && aligned16(g.A, g.lda, 4) && aligned16(g.Bm, g.ldb, 4);
            const int64_t tN128 = (g.N + 127) / 128;
            // 512 or more workgroups of 128 columns: a ring of five chunks;
            // 256 to 511 (fp32 4096^2: 1024 x 4096 products) in rounds of 256
            // more than 3/4 full: a ring of three, whose smaller register set
            // leaves room for two waves per SIMD.  Measured: 4096^2 0.680 ->
            // 0.661 ms against the LDS tiles; the ring of three lost on
            // 8192^2 (4.43 -> 5.17 ms) and on 384 workgroups (an update of
            // fp32 8192 x 2048: 144 -> 183 us, half the CUs running a second
            // round alone)
            if (g.a_lower) {
                const int64_t pairs = ((g.M + 63) / 64 + 1) / 2;
                if (lf && pairs * tN128 >= 512) return launch_lf32<5, 2, true>(g, st);
                const int64_t p128 = pairs * tN128;
                // (the triangular form there with 64 x 16 wave tiles: twice the
                // workgroups, two per CU; 0.659 -> 0.652 ms on 4096^2)
                if (lf && p128 >= 256 && 4 * p128 > 3 * 256 * ((p128 + 255) / 256))
                    return launch_lf32<3, 1, true, 2>(g, st);
                // 64 to 255: the same form (fp32 2048^2: 0.174 -> 0.167 ms,
                // 4096 x 2048: 0.443 -> 0.428 ms against the LDS tiles)
                if (lf && p128 >= 64 && p128 < 256) return launch_lf32<3, 1, true, 2>(g, st);
                // fewer workgroups: the LDS tile, 64 x 64 while that still
                // gives 512 folded workgroups
                if (pairs * ((g.N + 63) / 64) >= 512) return launch_tile<T, 64, 64, KT>(g, st);
            } else if (lf) {
                const int64_t t128 = ((g.M + 127) / 128) * tN128;
                if (g.M > 64 && t128 >= 512 && 4 * t128 >= 3 * 512 * ((t128 + 511) / 512))
                    return launch_lf32<5, 4, false>(g, st);
                // (the update there on 128 x 64 workgroups, 64 x 32 per wave,
                // two per CU: twice the workgroups; 0.649 -> 0.637 ms on 4096^2)
                if (g.M > 64 && t128 >= 256 && t128 < 512 && 4 * t128 > 3 * 256 * ((t128 + 255) / 256)) {
                    // K of 2048 and more: 64 x 64 per wave with K split over two
                    // waves per SIMD (eight-wave workgroups, the halves added
                    // through LDS) keeps two waves per SIMD on the larger wave
                    // tile: fp32 8192^2 4.27 -> 4.18 ms, 8192 x 4096 2.195 ->
                    // 2.162 ms, 4096^2 0.638 -> 0.634 ms; shorter K lost (the
                    // 1024 x 4096 x 1024 update 82 -> 89 us).  TRSM_LF32_KS sets
                    // the K bound (0: off)
                    const char *ek = std::getenv("TRSM_LF32_KS");
                    const int64_t kmin = ek ? std::atoll(ek) : 2048;
                    if (kmin > 0 && g.K >= kmin) return launch_lf32<2, 4, false, 1, 2>(g, st);
                    return launch_lf32<3, 2, false, 2>(g, st);
                }
                // 64 to 255: 128 x 32 workgroups (64 x 16 per wave, a ring of
                // four), four per tile (fp32 2048^2 0.174 -> 0.166 ms,
                // 4096 x 1024 0.330 -> 0.319 ms; with the triangular rule
                // above 2048^2 takes 0.159 ms)
                if (g.M > 64 && t128 >= 64 && t128 < 256) return launch_lf32<4, 1, false, 2>(g, st);
            }
        }
    }
    if constexpr (std::is_same<T, cplx32>::value) {
        bool taken = false;
        const hipError_t e = launch_c32_lf(g, st, taken);
        if (taken || e != hipSuccess) return e;
    }
    // Triangular solve products (folded pairs of row tiles) of fp64 and
    // complex fp64: the LDS-free forms below; without them, wider LDS tiles
    // once they give 512 folded workgroups, 64 x 128 for fp64 and 64 x 64 for
    // complex (measured on those tiles: fp64 8192^2 9.259 -> 9.218 ms, complex
    // 8192 x 2048 9.574 -> 9.457 ms), else 64 x 32.
    if (g.a_lower && !g.b_lower && g.batch <= 1) {
        const int64_t Mr = GemmTraits<T>::kCplx ? 2 * g.M : g.M;
        const int64_t pairs = ((Mr + 63) / 64 + 1) / 2;
        if constexpr (std::is_same<T, double>::value) {
            const bool lf = use_gemm_lf() && aligned16(g.A, g.lda, 8) && aligned16(g.Bm, g.ldb, 8);
            if (pairs * ((g.N + 127) / 128) >= 512) {
                if (lf) return launch_lf_tri(g, st);
                return launch_tile<T, 64, 128, KT>(g, st);
            }
            // 256 to 511 such workgroups (fp64 4096^2: 1024 x 4096 products,
            // one workgroup per CU): a ring of three, as for complex fp64
            // below; fp64 4096^2 1.372 -> 1.322 ms against the 64 x 32 LDS
            // tile (whole solves, same box)
            if (lf && pairs * ((g.N + 127) / 128) >= 256) return launch_lf_tri<3>(g, st);
            // fewer: 64 columns per workgroup (64 x 16 per wave, a ring of four)
            // while that gives 256 (fp64 4096 x 2048: 0.797 -> 0.767 ms)
            if (lf && pairs * ((g.N + 63) / 64) >= 256) return launch_lf_tri<4, 1>(g, st);
        }
        if constexpr (std::is_same<T, cplx>::value) {
            // the real view on the LDS-free kernel once the folded pairs give
            // 256 workgroups of 128 columns (64 x 32 per wave, a ring of
            // three chunks); TRSM_LF_CPLX_TRI=0 keeps the LDS tiles.
            // Measured (whole solves, two rounds on one box, against the
            // 64 x 64 LDS tile): complex 8192 x 2048 8.58-8.61 -> 8.48-8.50 ms,
            // 4096^2 4.44-4.45 -> 4.34-4.35 ms; rings of five (64 x 32) and
            // four (64 x 16 per wave, 512 workgroups) were within 1 % behind.
            const char *et = std::getenv("TRSM_LF_CPLX_TRI");
            if (use_gemm_lf() && !(et && et[0] == '0') && aligned16(g.A, g.lda, 16) &&
                aligned16(g.Bm, g.ldb, 16) && pairs * ((g.N + 127) / 128) >= 256)
                return launch_lf_tri_cplx<3, 2>(g, st);
            // (fewer: 64 x 16 per wave while that gives 256 workgroups;
            // complex 8192 x 1024 5.019 -> 4.910 ms, 4096 x 2048 2.585 -> 2.544)
            if (use_gemm_lf() && !(et && et[0] == '0') && aligned16(g.A, g.lda, 16) &&
                aligned16(g.Bm, g.ldb, 16) && pairs * ((g.N + 63) / 64) >= 256)
                return launch_lf_tri_cplx<4, 1>(g, st);
            if (pairs * ((g.N + 63) / 64) >= 512) return launch_tile<T, 64, 64, KT>(g, st);
        }
    }
    if (g.a_lower || g.b_lower) return launch_tile<T, 64, 32, KT>(g, st);
    if (g.batch <= 1) {
        const int64_t Mr = GemmTraits<T>::kCplx ? 2 * g.M : g.M;
        if constexpr (std::is_same<T, cplx>::value) {
            // real view 2M x N on 128 x 128 tiles without LDS, under the
            // fp64 rule (at least 512 tiles, rounds at least 3/4 full);
            // TRSM_LF_CPLX=0 keeps the LDS tiles (tuning)
            const int64_t t128 = ((Mr + 127) / 128) * ((g.N + 127) / 128);
            const char *ec = std::getenv("TRSM_LF_CPLX");
            if (use_gemm_lf() && !(ec && ec[0] == '0') && t128 >= 512 &&
                4 * t128 >= 3 * 512 * ((t128 + 511) / 512) && aligned16(g.A, g.lda, 16) &&
                aligned16(g.Bm, g.ldb, 16))
                return launch_lf_cplx(g, st);
            if (use_gemm_lf() && !(ec && ec[0] == '0') && Mr > 64 && use_lf_mid(t128) &&
                aligned16(g.A, g.lda, 16) && aligned16(g.Bm, g.ldb, 16))
                return launch_lf_cplx_n<3, 2>(g, st);
            if (use_gemm_lf() && !(ec && ec[0] == '0') && Mr > 64 && use_lf_low(t128) &&
                aligned16(g.A, g.lda, 16) && aligned16(g.Bm, g.ldb, 16))
                return launch_lf_cplx_n<4, 1>(g, st);
        }
        if constexpr (GemmTraits<T>::kCplx) {
            if (((Mr + 63) / 64) * ((g.N + 127) / 128) >= 2048) return launch_tile<T, 64, 128, KT>(g, st);
        } else if constexpr (sizeof(T) == 8) {
            // (16-byte aligned operands only: the dword-load form needs
            // all 256 VGPRs and runs one wave per SIMD)
            // (and more than 64 rows, which a 64-row tile already covers).
            // Its rounds of 512 tiles must also be at least 3/4 full: 585
            // tiles (fp64 1100 x 8300) leave a second round nearly empty and
            // ran 41.5 TFLOP/s where 64 x 64 tiles fill their rounds.
            const int64_t t128 = ((Mr + 127) / 128) * ((g.N + 127) / 128);
            if (Mr > 64 && t128 >= 512 && 4 * t128 >= 3 * 512 * ((t128 + 511) / 512) &&
                aligned16(g.A, g.lda, sizeof(T)) && aligned16(g.Bm, g.ldb, sizeof(T))) {
                if constexpr (std::is_same<T, double>::value) {
                    if (use_gemm_lf()) return launch_lf(g, st);
                }
                return launch_tile<T, 128, 128, KT>(g, st);
            }
            if constexpr (std::is_same<T, double>::value) {
                if (use_gemm_lf() && Mr > 64 && use_lf_mid(t128) && aligned16(g.A, g.lda, 8) &&
                    aligned16(g.Bm, g.ldb, 8))
                    return launch_lf_n<3, 2>(g, st);
                if (use_gemm_lf() && Mr > 64 && use_lf_low(t128) && aligned16(g.A, g.lda, 8) &&
                    aligned16(g.Bm, g.ldb, 8))
                    return launch_lf_n<4, 1>(g, st);
            }
            if (((Mr + 127) / 128) * ((g.N + 63) / 64) >= 2048) return launch_tile<T, 128, 64, KT>(g, st);
        }
        if (((Mr + 63) / 64) * ((g.N + 63) / 64) < 1024) return launch_tile<T, 64, 32, KT>(g, st);
        return launch_tile<T, 64, 64, KT>(g, st);
    }
    return launch_tile<T, 64, 32, KT>(g, st);  // batched: split-K chunks, other inversion products
}

// ---- split K: the reduction of the partial products -----------------------
template <typename T>
__device__ __forceinline__ T add_elem(T a, T b) {
    if constexpr (GemmTraits<T>::kCplx) return T{a.re + b.re, a.im + b.im};
    else return a + b;
}

// out(i, j) = gamma * sum_s part_s(i, j) + beta * C(i, j); one column per
// blockIdx.y, rows across the threads (coalesced over every operand).
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    int64_t M, int parts, const T *__restrict__ part, int64_t pstride, const T *__restrict__ C,
    int64_t ldc, T *__restrict__ D, int64_t ldd, T *__restrict__ D2, int64_t ldd2, int64_t split,
    Scalar beta, Scalar gamma, int has_c) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M) return;
    const int64_t j = blockIdx.y;
    const T *src = part + i + j * M;
    T s = src[0];
    for (int t = 1; t < parts; ++t) s = add_elem<T>(s, src[t * pstride]);
    T out = Elem<T>::mul(Elem<T>::from(gamma), s);
    if (has_c) out = add_elem<T>(out, Elem<T>::mul(Elem<T>::from(beta), C[i + j * ldc]));
    if (i < split) D2[i + j * ldd2] = out;
    else D[i + j * ldd] = out;
}

template <typename T>
hipError_t splitk_reduce_t(const GemmDesc &g, int parts, const void *partial, hipStream_t st) {
    const int64_t gx = (g.M + 255) / 256;
    if (g.N > 65535 || gx > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int has_c = (g.C != nullptr) && (g.beta.re != 0.0 || g.beta.im != 0.0);
    T *D = static_cast<T *>(g.D);
    T *D2 = g.D2 ? static_cast<T *>(g.D2) : D;
    hipLaunchKernelGGL((splitk_reduce_kernel<T>), dim3((unsigned)gx, (unsigned)g.N), dim3(256), 0,
                       st, g.M, parts, static_cast<const T *>(partial), g.M * g.N,
                       static_cast<const T *>(g.C), g.ldc, D, g.ldd, D2,
                       g.D2 ? g.ldd2 : g.ldd, g.D2 ? g.split : (int64_t)0, g.beta, g.gamma, has_c);
    return hipGetLastError();
}

}  // namespace

int gemm_splitk_parts(int dtype, int64_t M, int64_t N, int64_t K, int64_t target_workgroups) {
    // the reduction puts one column per grid row (at most 65535)
    if (M <= 0 || N <= 0 || N > 65535 || K <= 0 || target_workgroups <= 0) return 1;
    const int64_t Mr = (dtype == C64F || dtype == C32F) ? 2 * M : M;
    const int64_t tiles = ((Mr + 63) / 64) * ((N + 31) / 32);
    int64_t parts = 1;
    while (2 * parts * tiles <= target_workgroups && K % (2 * parts * kSplitKMinChunk) == 0 &&
           2 * parts * M * N <= kSplitKMaxElems)
        parts *= 2;
    return (int)parts;
}

hipError_t gemm_splitk_launch(int dtype, const GemmDesc &g, int parts, void *partial,
                              hipStream_t stream) {
    if (parts <= 1) return gemm_launch(dtype, g, stream);
    if (use_ks(dtype, g)) return launch_ks(dtype, g, parts, stream);
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    if (g.batch > 1 || g.K % parts != 0 || partial == nullptr ||
        (int64_t)parts * g.M * g.N > kSplitKMaxElems)
        return hipErrorInvalidValue;
    const int64_t kc = g.K / parts;
    GemmDesc c{};
    c.M = g.M;
    c.N = g.N;
    c.K = kc;
    c.A = g.A;
    c.lda = g.lda;
    c.Bm = g.Bm;
    c.ldb = g.ldb;
    c.C = nullptr;
    c.ldc = g.M;
    c.D = partial;
    c.ldd = g.M;
    c.beta = Scalar{0.0, 0.0};
    c.gamma = Scalar{1.0, 0.0};
    c.a_lower = g.a_lower;
    c.batch = parts;
    c.binner = 1;
    c.sAo = kc * g.lda;  // chunk s: columns [s*kc, (s+1)*kc) of A
    c.sBo = kc;          //          rows [s*kc, (s+1)*kc) of Bm
    c.sDo = g.M * g.N;
    c.sKo = kc;          // triangular A: chunk s skips the K tiles right of the diagonal
    hipError_t e = gemm_launch(dtype, c, stream);
    if (e != hipSuccess) return e;
    switch (dtype) {
        case R32F: return splitk_reduce_t<float>(g, parts, partial, stream);
        case R64F: return splitk_reduce_t<double>(g, parts, partial, stream);
        case C64F: return splitk_reduce_t<cplx>(g, parts, partial, stream);
        case C32F: return splitk_reduce_t<cplx32>(g, parts, partial, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t gemm_launch(int dtype, const GemmDesc &g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    if (g.a_lower && g.b_lower) return hipErrorInvalidValue;
    // Buffer loads take 32-bit offsets from a tile's first element: they
    // reach the 32 (fp32) or 16 K columns of an A tile and the up to 128
    // columns of a Bm tile only while those span less than 2 GB.  Beyond
    // that the 64 x 32 tile runs with 64-bit addresses.
    const int64_t es = (int64_t)dtype_size(dtype);
    if (g.lda > (0x7fffffffLL - 4096) / (es * 32) || g.ldb > (0x7fffffffLL - 4096) / (es * 128)) {
        switch (dtype) {
            case R32F: return launch_wide<float, 32>(g, stream);
            case R64F: return launch_wide<double, 16>(g, stream);
            case C64F: return launch_wide<cplx, 16>(g, stream);
            case C32F: return launch_wide<cplx32, 32>(g, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (dtype) {
        case R32F: return launch_sized<float, 32>(g, stream);
        case R64F: return launch_sized<double, 16>(g, stream);
        case C64F: return launch_sized<cplx, 16>(g, stream);
        case C32F: return launch_sized<cplx32, 32>(g, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace trsm
