// Device arithmetic on the element types (float, double, cplx, cplx32).
// Complex products are written out in real fused multiply-adds; no operand is
// conjugated.
#pragma once

#include "trsm_internal.h"

namespace trsm {

template <typename T> struct Elem;

template <> struct Elem<float> {
    using Real = float;
    static constexpr int kDType = R32F;
    __device__ __forceinline__ static float zero() { return 0.0f; }
    __device__ __forceinline__ static float one() { return 1.0f; }
    __device__ __forceinline__ static float from(Scalar s) { return (float)s.re; }
    __device__ __forceinline__ static float mul(float a, float b) { return a * b; }
    // b - l*x
    __device__ __forceinline__ static float msub(float b, float l, float x) {
        return __builtin_fmaf(-l, x, b);
    }
    __device__ __forceinline__ static float recip(float d) { return 1.0f / d; }
    __device__ __forceinline__ static float sel(bool c, float a, float b) { return c ? a : b; }
};

template <> struct Elem<double> {
    using Real = double;
    static constexpr int kDType = R64F;
    __device__ __forceinline__ static double zero() { return 0.0; }
    __device__ __forceinline__ static double one() { return 1.0; }
    __device__ __forceinline__ static double from(Scalar s) { return s.re; }
    __device__ __forceinline__ static double mul(double a, double b) { return a * b; }
    __device__ __forceinline__ static double msub(double b, double l, double x) {
        return __builtin_fma(-l, x, b);
    }
    __device__ __forceinline__ static double recip(double d) { return 1.0 / d; }
    __device__ __forceinline__ static double sel(bool c, double a, double b) { return c ? a : b; }
};

template <> struct Elem<cplx> {
    using Real = double;
    static constexpr int kDType = C64F;
    __device__ __forceinline__ static cplx zero() { return cplx{0.0, 0.0}; }
    __device__ __forceinline__ static cplx one() { return cplx{1.0, 0.0}; }
    __device__ __forceinline__ static cplx from(Scalar s) { return cplx{s.re, s.im}; }
    __device__ __forceinline__ static cplx mul(cplx a, cplx b) {
        return cplx{__builtin_fma(a.re, b.re, -a.im * b.im),
                    __builtin_fma(a.re, b.im, a.im * b.re)};
    }
    // b - l*x = (b.re - l.re x.re + l.im x.im) + (b.im - l.re x.im - l.im x.re) i
    __device__ __forceinline__ static cplx msub(cplx b, cplx l, cplx x) {
        double r = __builtin_fma(-l.re, x.re, b.re);
        r = __builtin_fma(l.im, x.im, r);
        double i = __builtin_fma(-l.re, x.im, b.im);
        i = __builtin_fma(-l.im, x.re, i);
        return cplx{r, i};
    }
    // 1/d; a real divisor (imaginary part 0, the case of every generated
    // input) gives the exactly rounded real reciprocal.
    __device__ __forceinline__ static cplx recip(cplx d) {
        if (d.im == 0.0) return cplx{1.0 / d.re, 0.0};
        double den = d.re * d.re + d.im * d.im;
        return cplx{d.re / den, -d.im / den};
    }
    // c ? a : b, part by part (keeps the values in registers)
    __device__ __forceinline__ static cplx sel(bool c, cplx a, cplx b) {
        return cplx{c ? a.re : b.re, c ? a.im : b.im};
    }
};

template <> struct Elem<cplx32> {
    using Real = float;
    static constexpr int kDType = C32F;
    __device__ __forceinline__ static cplx32 zero() { return cplx32{0.0f, 0.0f}; }
    __device__ __forceinline__ static cplx32 one() { return cplx32{1.0f, 0.0f}; }
    __device__ __forceinline__ static cplx32 from(Scalar s) { return cplx32{(float)s.re, (float)s.im}; }
    __device__ __forceinline__ static cplx32 mul(cplx32 a, cplx32 b) {
        return cplx32{__builtin_fmaf(a.re, b.re, -a.im * b.im),
                      __builtin_fmaf(a.re, b.im, a.im * b.re)};
    }
    __device__ __forceinline__ static cplx32 msub(cplx32 b, cplx32 l, cplx32 x) {
        float r = __builtin_fmaf(-l.re, x.re, b.re);
        r = __builtin_fmaf(l.im, x.im, r);
        float i = __builtin_fmaf(-l.re, x.im, b.im);
        i = __builtin_fmaf(-l.im, x.re, i);
        return cplx32{r, i};
    }
    __device__ __forceinline__ static cplx32 recip(cplx32 d) {
        if (d.im == 0.0f) return cplx32{1.0f / d.re, 0.0f};
        float den = d.re * d.re + d.im * d.im;
        return cplx32{d.re / den, -d.im / den};
    }
    __device__ __forceinline__ static cplx32 sel(bool c, cplx32 a, cplx32 b) {
        return cplx32{c ? a.re : b.re, c ? a.im : b.im};
    }
};

}  // namespace trsm
