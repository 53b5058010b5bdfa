// Small memory kernels around the solve: zeroing B (alpha == 0, where the
// result is X = 0 and A is not read), copying one panel of B into the
// panel buffer that the first diagonal-block solve reads, and the index
// reflections that bring the other TRSM variants to the left-lower form.
#include "scalar_ops.h"
#include "buffer_ops.h"

#include <cstdint>
#include <type_traits>

namespace trsm {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void fill_zero_kernel(int64_t m, int64_t n, T *__restrict__ B,
                                                        int64_t ldb, int64_t strideB,
                                                        int64_t batch) {
    const int64_t total = m * n * batch;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e % m;
        const int64_t rest = e / m;
        const int64_t j = rest % n;
        const int64_t p = rest / n;
        B[p * strideB + i + j * ldb] = Elem<T>::zero();
    }
}

// dst(i, j) = src(i, j) for a rows x n column-major panel.  Thread t of a
// workgroup takes V consecutive rows (one 16-byte access when VEC, else one
// element) of column t / tpc, with tpc threads per column (64, 128 or 256,
// the fewest that cover the rows in one pass where possible), so a short
// panel still keeps every lane busy.  Each thread copies CW columns
// cpw = 256 / tpc apart, all loads before the stores, and the workgroups
// stride over the column groups.  No 64-bit division per element.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void copy_panel_kernel(int64_t rows, int64_t n,
                                                         const T *__restrict__ src, int64_t lds,
                                                         T *__restrict__ dst, int64_t ldd, int tpc) {
    using W = typename std::conditional<VEC, u4v, T>::type;
    constexpr int V = (int)(sizeof(W) / sizeof(T));
    constexpr int CW = 4;
    const int t = threadIdx.x;
    const int cpw = 256 / tpc;
    const int64_t i = ((int64_t)blockIdx.x * tpc + (t % tpc)) * V;
    if (i >= rows) return;
    const int64_t group = (int64_t)cpw * CW;  // columns per workgroup and pass
    for (int64_t j0 = (int64_t)blockIdx.y * group + t / tpc; j0 < n; j0 += (int64_t)gridDim.y * group) {
        W v[CW];
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const int64_t j = j0 + (int64_t)c * cpw;
            if (j < n) v[c] = *reinterpret_cast<const W *>(src + i + j * lds);
        }
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const int64_t j = j0 + (int64_t)c * cpw;
            if (j < n) *reinterpret_cast<W *>(dst + i + j * ldd) = v[c];
        }
    }
}

// dst(i, j) = f(src(a, b)) for an R x C dst, with a = revR ? R-1-i : i and
// b = revC ? C-1-j : j; src(a, b) is src[a + b*lds], or src[b + a*lds] when
// trans (src then holds the transposed matrix); f conjugates when conj.
// lower: only i >= j is written (and read); unit: dst(i, i) = 1 without
// reading src.  32 x 32 tiles of dst per workgroup; the transposing form
// goes through LDS so that both the reads and the writes are coalesced.
template <typename T>
__device__ __forceinline__ T conj_if(T v, int) { return v; }
template <>
__device__ __forceinline__ cplx conj_if<cplx>(cplx v, int c) { return c ? cplx{v.re, -v.im} : v; }
template <>
__device__ __forceinline__ cplx32 conj_if<cplx32>(cplx32 v, int c) { return c ? cplx32{v.re, -v.im} : v; }

template <typename T>
__global__ __launch_bounds__(256) void transform_kernel(int64_t R, int64_t C,
                                                        const T *__restrict__ src, int64_t lds,
                                                        T *__restrict__ dst, int64_t ldd, int revR,
                                                        int revC, int trans, int conj, int lower,
                                                        int unit) {
    __shared__ T tile[32][33];
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    const int64_t i0 = (int64_t)blockIdx.x * 32;
    auto wanted = [&](int64_t i, int64_t j) { return i < R && j < C && (!lower || i >= j); };
    auto put = [&](int64_t i, int64_t j, T v) {
        dst[i + j * ldd] = (unit && i == j) ? Elem<T>::one() : conj_if<T>(v, conj);
    };
    // column tiles in a grid-stride loop: gridDim.y is capped at 65535, and
    // every thread of the block runs the same iterations (uniform bounds)
    const int64_t ntj = (C + 31) / 32;
    for (int64_t jt = blockIdx.y; jt < ntj; jt += gridDim.y) {
        const int64_t j0 = jt * 32;
        if (lower && i0 + 31 < j0) break;  // this and later tiles lie above the diagonal
        if (!trans) {
            for (int jj = ty; jj < 32; jj += 8) {
                const int64_t i = i0 + tx, j = j0 + jj;
                if (!wanted(i, j)) continue;
                const int64_t a = revR ? R - 1 - i : i, b = revC ? C - 1 - j : j;
                put(i, j, (unit && i == j) ? Elem<T>::one() : src[a + b * lds]);
            }
            continue;
        }
        // read src(b, a) with consecutive threads on consecutive b (src rows)
        for (int ii = ty; ii < 32; ii += 8) {
            const int64_t i = i0 + ii, j = j0 + tx;
            if (wanted(i, j) && !(unit && i == j)) {
                const int64_t a = revR ? R - 1 - i : i, b = revC ? C - 1 - j : j;
                tile[ii][tx] = src[b + a * lds];
            }
        }
        __syncthreads();
        for (int jj = ty; jj < 32; jj += 8) {
            const int64_t i = i0 + tx, j = j0 + jj;
            if (wanted(i, j)) put(i, j, tile[tx][jj]);
        }
        __syncthreads();  // the tile is reused by the next column tile
    }
}

inline unsigned grid_for(int64_t total) {
    int64_t g = (total + 255) / 256;
    if (g > 65536) g = 65536;  // grid-stride loops cover the rest
    return (unsigned)(g < 1 ? 1 : g);
}

template <typename T>
hipError_t fill_t(int64_t m, int64_t n, void *B, int64_t ldb, int64_t sB, int64_t batch,
                  hipStream_t st) {
    const int64_t total = m * n * batch;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL((fill_zero_kernel<T>), dim3(grid_for(total)), dim3(256), 0, st, m, n,
                       static_cast<T *>(B), ldb, sB, batch);
    return hipGetLastError();
}

template <typename T>
hipError_t copy_t(int64_t rows, int64_t n, const void *src, int64_t lds, void *dst, int64_t ldd,
                  hipStream_t st) {
    if (rows <= 0 || n <= 0) return hipSuccess;
    constexpr int64_t V = 16 / (int64_t)sizeof(T);
    const bool vec = V > 1 && rows % V == 0 && lds % V == 0 && ldd % V == 0 &&
                     reinterpret_cast<uintptr_t>(src) % 16 == 0 && reinterpret_cast<uintptr_t>(dst) % 16 == 0;
    const int64_t per = vec ? (rows + V - 1) / V : rows;  // threads per column
    const int tpc = per <= 64 ? 64 : per <= 128 ? 128 : 256;
    const int64_t gx = (per + tpc - 1) / tpc;
    const int64_t group = (256 / tpc) * 4;
    int64_t gy = (n + group - 1) / group;
    if (gy > 65535) gy = 65535;  // the kernel strides over the rest
    if (gx > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    if (vec)
        hipLaunchKernelGGL((copy_panel_kernel<T, true>), grid, dim3(256), 0, st, rows, n,
                           static_cast<const T *>(src), lds, static_cast<T *>(dst), ldd, tpc);
    else
        hipLaunchKernelGGL((copy_panel_kernel<T, false>), grid, dim3(256), 0, st, rows, n,
                           static_cast<const T *>(src), lds, static_cast<T *>(dst), ldd, tpc);
    return hipGetLastError();
}

template <typename T>
hipError_t transform_t(int64_t R, int64_t C, const void *src, int64_t lds, void *dst, int64_t ldd,
                       const Reflect &f, hipStream_t st) {
    if (R <= 0 || C <= 0) return hipSuccess;
    const int64_t gx = (R + 31) / 32;
    const int64_t gy = (C + 31) / 32 < 65535 ? (C + 31) / 32 : 65535;  // the kernel strides over the rest
    if (gx > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((transform_kernel<T>), dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st, R,
                       C, static_cast<const T *>(src), lds, static_cast<T *>(dst), ldd, f.revR,
                       f.revC, f.trans, f.conj, f.lower, f.unit);
    return hipGetLastError();
}

}  // namespace

hipError_t transform_launch(int dtype, int64_t R, int64_t C, const void *src, int64_t lds,
                            void *dst, int64_t ldd, const Reflect &f, hipStream_t stream) {
    switch (dtype) {
        case R32F: return transform_t<float>(R, C, src, lds, dst, ldd, f, stream);
        case R64F: return transform_t<double>(R, C, src, lds, dst, ldd, f, stream);
        case C64F: return transform_t<cplx>(R, C, src, lds, dst, ldd, f, stream);
        case C32F: return transform_t<cplx32>(R, C, src, lds, dst, ldd, f, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t fill_zero_launch(int dtype, int64_t m, int64_t n, void *B, int64_t ldb,
                            int64_t strideB, int64_t batch, hipStream_t stream) {
    switch (dtype) {
        case R32F: return fill_t<float>(m, n, B, ldb, strideB, batch, stream);
        case R64F: return fill_t<double>(m, n, B, ldb, strideB, batch, stream);
        case C64F: return fill_t<cplx>(m, n, B, ldb, strideB, batch, stream);
        // complex fp32 is 8 bytes: zero bits and a bit copy, as for fp64
        case C32F: return fill_t<double>(m, n, B, ldb, strideB, batch, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t copy_panel_launch(int dtype, int64_t rows, int64_t n, const void *src, int64_t lds,
                             void *dst, int64_t ldd, hipStream_t stream) {
    switch (dtype) {
        case R32F: return copy_t<float>(rows, n, src, lds, dst, ldd, stream);
        case R64F: return copy_t<double>(rows, n, src, lds, dst, ldd, stream);
        case C64F: return copy_t<cplx>(rows, n, src, lds, dst, ldd, stream);
        case C32F: return copy_t<double>(rows, n, src, lds, dst, ldd, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace trsm
