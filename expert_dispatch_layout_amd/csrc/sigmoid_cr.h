// Correctly rounded binary32 logistic sigmoid on gfx950.
//
// The sigmoid of the TensorRT-LLM RoutingKernel.cuh helpers (sigmoid_accurate) is the real
// function 1/(1+exp(-x)); its rounding is not fixed there.  Selection keys are built from it, so
// this library returns the correctly rounded value (round to nearest even, subnormals kept),
// which is unique and therefore reproducible on any machine.
//
// Method (Ziv's onion-peeling strategy):
//   fast path  evaluate in binary64 (relative error below 2^-48, see sigmoid_f64); widen by
//              2^-44 and accept when both ends round to the same binary32 value;
//   slow path  evaluate in double-double arithmetic (Dekker's two-sum / two-product) to about
//              2^-90 relative and decide the rounding from the double-double value, again with
//              an interval check.  The exponential uses exp(t) = exp(t/2^12)^(2^12): an exact
//              power-of-two scaling, a degree-16 Taylor polynomial and twelve squarings, so no
//              split constant of ln 2 is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mep {

struct dd_t {
    double hi, lo;
};

__device__ __forceinline__ dd_t dd_two_sum(double a, double b) {
    double s = a + b;
    double bb = s - a;
    double e = (a - (s - bb)) + (b - bb);
    return {s, e};
}

// requires |a| >= |b| (or a == 0)
__device__ __forceinline__ dd_t dd_quick_two_sum(double a, double b) {
    double s = a + b;
    return {s, b - (s - a)};
}

__device__ __forceinline__ dd_t dd_two_prod(double a, double b) {
    double p = a * b;
    return {p, __fma_rn(a, b, -p)};
}

__device__ __forceinline__ dd_t dd_add(dd_t a, dd_t b) {
    dd_t s = dd_two_sum(a.hi, b.hi);
    dd_t t = dd_two_sum(a.lo, b.lo);
    s.lo += t.hi;
    s = dd_quick_two_sum(s.hi, s.lo);
    s.lo += t.lo;
    return dd_quick_two_sum(s.hi, s.lo);
}

__device__ __forceinline__ dd_t dd_mul(dd_t a, dd_t b) {
    dd_t p = dd_two_prod(a.hi, b.hi);
    p.lo += a.hi * b.lo + a.lo * b.hi;
    return dd_quick_two_sum(p.hi, p.lo);
}

__device__ __forceinline__ dd_t dd_mul_d(dd_t a, double b) {
    dd_t p = dd_two_prod(a.hi, b);
    p.lo += a.lo * b;
    return dd_quick_two_sum(p.hi, p.lo);
}

__device__ __forceinline__ dd_t dd_div_d(dd_t a, double b) {
    double q1 = a.hi / b;
    dd_t p = dd_two_prod(q1, b);
    double r = ((a.hi - p.hi) - p.lo) + a.lo;
    return dd_quick_two_sum(q1, r / b);
}

// 1 / a for a >= 1
__device__ __forceinline__ dd_t dd_recip(dd_t a) {
    double y = 1.0 / a.hi;
    // residual 1 - a*y in double-double, then one Newton correction
    dd_t ay = dd_mul_d(a, y);
    dd_t res = dd_add(dd_t{1.0, 0.0}, dd_t{-ay.hi, -ay.lo});
    dd_t corr = dd_mul_d(res, y);
    return dd_add(dd_t{y, 0.0}, corr);
}

// exp(t) for |t| <= 128 in double-double.
__device__ __noinline__ dd_t dd_exp(double t) {
    double u = t * 0x1p-12;  // exact
    dd_t p = {1.0, 0.0};
    for (int k = 16; k >= 1; --k) {
        p = dd_div_d(dd_mul_d(p, u), (double)k);
        p = dd_add(dd_t{1.0, 0.0}, p);
    }
    for (int i = 0; i < 12; ++i) p = dd_mul(p, p);
    return p;
}

// Correct binary32 rounding (nearest, ties to even) of a non-negative double-double value.
__device__ __forceinline__ float dd_round_f32(dd_t v) {
    float f = (float)v.hi;
    double fd = (double)f;
    if (fd == v.hi) return f;
    uint32_t fb = __float_as_uint(f);
    float g = (v.hi > fd) ? __uint_as_float(fb + 1u) : __uint_as_float(fb - 1u);
    double mid = 0.5 * (fd + (double)g);  // exact: both are binary32 neighbours
    if (v.hi != mid || v.lo == 0.0) return f;
    float up = fd > (double)g ? f : g;
    float down = fd > (double)g ? g : f;
    return v.lo > 0.0 ? up : down;
}

__device__ __noinline__ float sigmoid_cr_slow(float x) {
    if (x != x) return x;
    // sigmoid(x) < e^x <= e^-104 < 2^-150 rounds to 0; 1 - sigmoid(x) < e^-x <= e^-17.5 < 2^-25
    // rounds to 1.
    if (x <= -104.0f) return 0.0f;
    if (x >= 17.5f) return 1.0f;
    dd_t e = dd_exp(-(double)x);
    dd_t s = dd_recip(dd_add(dd_t{1.0, 0.0}, e));
    double tol = s.hi * 0x1p-80;
    float lo = dd_round_f32(dd_quick_two_sum(s.hi, s.lo - tol));
    float hi = dd_round_f32(dd_quick_two_sum(s.hi, s.lo + tol));
    if (lo == hi) return lo;
    return dd_round_f32(s);
}

// A binary64 constant placed in scalar registers where it is used.  The empty volatile asm keeps
// the compiler from hoisting the constant out of loops into vector registers (where, under
// register pressure, it would be spilled and reloaded from scratch memory instead).
__device__ __forceinline__ double sreg(double v) {
    asm volatile("" : "+s"(v));
    return v;
}

// Coefficients of 2^f = e^(f ln 2) for |f| <= 1/2: the Taylor series to degree 13, (ln 2)^k / k!
// rounded to binary64, highest degree first (the constant term 1 is added separately).  The
// truncation error is below 2^-56 for |f ln 2| <= 0.35.
constexpr int kExp2Terms = 13;
constexpr double kExp2Coef[kExp2Terms] = {
    0x1.816193166d0f9p-40, 0x1.c3bd650fc2986p-36, 0x1.e8cac7351bb25p-32, 0x1.e4cf5158b8ecap-28,
    0x1.b5253d395e7c4p-24, 0x1.62c0223a5c824p-20, 0x1.ffcbfc588b0c7p-17, 0x1.430912f86c787p-13,
    0x1.5d87fe78a6731p-10, 0x1.3b2ab6fba4e77p-7,  0x1.c6b08d704a0c0p-5,  0x1.ebfbdff82c58fp-3,
    0x1.62e42fefa39efp-1};

// Coefficient source: scalar-register constants (the default).
struct Exp2CoefConst {
    __device__ __forceinline__ double operator()(int i) const { return sreg(kExp2Coef[i]); }
};

// 2^y in binary64 for |y| <= 1100.  y = n + f with n = rint(y) and |f| <= 1/2 (exact); 2^f by
// the series above in Horner form, then an exact scaling by 2^n.  Relative error below 2^-51.
// `coef(i)` supplies kExp2Coef[i].  FIRST > 0 drops the FIRST highest-degree terms: FIRST = 5
// keeps degree 8, whose truncation error is below 2^-31 (enough where only about 2^-30 relative
// accuracy is needed, with fewer constants to hold).
template <int FIRST = 0, typename C>
__device__ __forceinline__ double exp2_f64_c(double y, C coef) {
    const double n = __builtin_rint(y);
    const double f = y - n;
    double p = coef(FIRST);
#pragma unroll
    for (int i = FIRST + 1; i < kExp2Terms; ++i) p = __fma_rn(p, f, coef(i));
    p = __fma_rn(p, f, 1.0);
    return __builtin_amdgcn_ldexp(p, (int)n);
}

__device__ __forceinline__ double exp2_f64(double y) { return exp2_f64_c(y, Exp2CoefConst{}); }

// 1/d for a positive normal binary64 d whose reciprocal is normal: the hardware reciprocal
// refined by two Newton steps
// r <- r + r (1 - d r), each of which squares the relative error; result within 2^-52.
__device__ __forceinline__ double recip_f64(double d) {
    double r = __builtin_amdgcn_rcp(d);
    double e = __fma_rn(-d, r, 1.0);
    r = __fma_rn(r, e, r);
    e = __fma_rn(-d, r, 1.0);
    return __fma_rn(r, e, r);
}

// e^t in binary64 for t <= 0 (softmax terms): 2^(t log2 e), with relative error below
// (|t| + 4) 2^-53 (the rounding of t log2 e dominates for large |t|); 0 or a subnormal below
// about e^-734.
__device__ __forceinline__ double exp_neg_f64(double t) {
    const double y = fmax(t * 0x1.71547652b82fep+0, -1060.0);
    return exp2_f64(y);
}

// sigma(x) = 1 / (1 + 2^y), y = -x log2(e), in binary64 with relative error below 2^-48.
// y is formed as x * C_hi + x * C_lo with C_hi = -log2(e) rounded to 29 significant bits (so the
// first product of a binary32 x is exact) and C_lo the binary64 remainder; y is clamped to
// [-1060, 1000], where sigma is 1 or far below the smallest binary32 subnormal either way.
template <int FIRST = 0, typename C>
__device__ __forceinline__ double sigmoid_f64_c(float x, C coef) {
    const double xd = (double)x;
    double y = __fma_rn(xd, 0x1.a8fa03d1105e0p-29, xd * -0x1.7154766p+0);
    y = fmin(fmax(y, -1060.0), 1000.0);
    return recip_f64(1.0 + exp2_f64_c<FIRST>(y, coef));
}

__device__ __forceinline__ double sigmoid_f64(float x) { return sigmoid_f64_c(x, Exp2CoefConst{}); }

// sigma(x) in binary64 with relative error below 2^-30: the degree-8 exponential.  For routing
// weights, which are compared at 1e-6 relative, not for selection keys.
__device__ __forceinline__ double sigmoid_f64_weight(float x) { return sigmoid_f64_c<5>(x, Exp2CoefConst{}); }

__device__ __forceinline__ float sigmoid_cr(float x) {
    const double s = sigmoid_f64(x);
    const double tol = s * 0x1p-44;
    float lo = (float)(s - tol);
    float hi = (float)(s + tol);
    if (lo == hi) return lo;
    return sigmoid_cr_slow(x);
}

// The fast path alone: `ok` is false when the interval test cannot decide the binary32
// rounding (about one value in 2^19); the caller then takes the exact path.
template <typename C>
__device__ __forceinline__ float sigmoid_cr_fast_c(float x, bool& ok, C coef) {
    const double s = sigmoid_f64_c(x, coef);
    const double tol = s * 0x1p-44;
    const float lo = (float)(s - tol);
    const float hi = (float)(s + tol);
    ok = lo == hi;
    return lo;
}

__device__ __forceinline__ float sigmoid_cr_fast(float x, bool& ok) {
    return sigmoid_cr_fast_c(x, ok, Exp2CoefConst{});
}

}  // namespace mep
