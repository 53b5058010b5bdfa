// Raw buffer loads for gfx950 kernels: a load at or past the end of the
// described range returns zero without a branch, so ragged edges cost no
// control flow.  Internal to the library.
#pragma once

#include <type_traits>

#include "trsm_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trsm {

typedef unsigned u4v __attribute__((ext_vector_type(4)));

// Raw buffer resource of a gfx9-family part (gfx950): base address, no
// stride, a byte range (loads at or past it return 0), 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint32_t n =
        bytes >= 0xffffffffLL ? 0xffffffffu : (bytes <= 0 ? 0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             0x00020000);
}

// 16 bytes at byte offset `off`.  VEC: the address is 16-byte aligned and
// one 16-byte load is used; otherwise four dword loads (every element type
// here is at least dword aligned).  VEC is a template parameter on purpose:
// with a run-time choice the two paths meet in a register copy, and the copy
// makes the compiler wait for the load at once, which defeats prefetching.
template <bool VEC>
__device__ __forceinline__ u4v ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (VEC) {
        return __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    } else {
        u4v v;
        v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        v[1] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4, 0, 0);
        v[2] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 8, 0, 0);
        v[3] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 12, 0, 0);
        return v;
    }
}

// 16 bytes at byte offset `off` from `base` through 64-bit global
// addresses, for operands whose leading dimension puts a tile's offsets past
// what a 32-bit buffer offset reaches.  Each dword is read only when it lies
// inside [0, lim) bytes from base, and is zero otherwise (no memory access),
// which is the same contract as a raw buffer load with range lim.
__device__ __forceinline__ u4v ld16_wide(const char *base, int64_t off, int64_t lim) {
    u4v v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int64_t o = off + 4 * d;
        v[d] = (o + 4 <= lim) ? *reinterpret_cast<const unsigned *>(base + o) : 0u;
    }
    return v;
}

// N consecutive elements of T at byte offset `off` into dst, as 16-byte
// loads where N * sizeof(T) allows it and dword loads otherwise.
template <typename T, int N, bool VEC>
__device__ __forceinline__ void ld_elems(__amdgpu_buffer_rsrc_t r, uint32_t off, T (&dst)[N]) {
    constexpr int NB = N * (int)sizeof(T);
    static_assert(NB % 4 == 0, "dword multiple");
    if constexpr (NB % 16 == 0) {
        constexpr int PER = 16 / (int)sizeof(T);
#pragma unroll
        for (int q = 0; q < NB / 16; ++q) {
            const u4v v = ld16<VEC>(r, off + 16 * q);
            // Bit-cast the whole vector to a vector of T and index that: a
            // bit cast of each u4v element on its own was compiled as a
            // repeat of element 0 (seen with hipcc for gfx950).
            if constexpr (std::is_same<T, cplx32>::value) {
                typedef float f4t __attribute__((ext_vector_type(4)));
                const f4t w = __builtin_bit_cast(f4t, v);
                dst[q * 2] = cplx32{w[0], w[1]};
                dst[q * 2 + 1] = cplx32{w[2], w[3]};
            } else if constexpr (sizeof(T) == 4) {
                typedef T v4t __attribute__((ext_vector_type(4)));
                const v4t w = __builtin_bit_cast(v4t, v);
#pragma unroll
                for (int e = 0; e < PER; ++e) dst[q * PER + e] = w[e];
            } else if constexpr (sizeof(T) == 8) {
                typedef T v2t __attribute__((ext_vector_type(2)));
                const v2t w = __builtin_bit_cast(v2t, v);
#pragma unroll
                for (int e = 0; e < PER; ++e) dst[q * PER + e] = w[e];
            } else {
                dst[q] = __builtin_bit_cast(T, v);
            }
        }
    } else {
        unsigned w[NB / 4];
#pragma unroll
        for (int q = 0; q < NB / 4; ++q)
            w[q] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * q, 0, 0);
        __builtin_memcpy(dst, w, NB);
    }
}

}  // namespace trsm
