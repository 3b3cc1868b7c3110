// Shared device types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wk {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Exact unsigned division n / d for n < 2^24 and 1 <= d < 2^16:
// with mul = ceil(2^40 / d), n * mul / 2^40 exceeds n / d by less than
// n / 2^40 < 1 / d, which never crosses the next integer.
struct DivU {
    uint64_t mul;
    uint32_t d;
};

static inline DivU make_divu(uint32_t d) {
    DivU r;
    r.d = d;
    r.mul = ((uint64_t(1) << 40) + d - 1) / d;
    return r;
}

__device__ __forceinline__ uint32_t divu(uint32_t n, const DivU &v) {
    return uint32_t((uint64_t(n) * v.mul) >> 40);
}

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions (1964),
// formula 7.1.26 (Hastings' rational approximation): for x >= 0,
//   erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
//   t = 1 / (1 + p x),
// with |error| <= 1.5e-7; odd symmetry gives x < 0.  Two transcendental
// instructions (reciprocal, exp2) and eight FMA-class operations.
__device__ __forceinline__ float erf_as(float x) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
    float poly = fmaf(1.061405429f, t, -1.453152027f);
    poly = fmaf(poly, t, 1.421413741f);
    poly = fmaf(poly, t, -0.284496736f);
    poly = fmaf(poly, t, 0.254829592f);
    poly *= t;
    const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
    return copysignf(1.0f - poly * e, x);
}

// Exact GELU, the error-function form: 0.5 z (1 + erf(z / sqrt 2)).
__device__ __forceinline__ float gelu_erf(float z) {
    return 0.5f * z * (1.0f + erf_as(z * 0.70710678118654752f));
}

}  // namespace wk
