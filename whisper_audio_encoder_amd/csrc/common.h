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

// Exact GELU, the error-function form: gelu(z) = z Phi(z), Phi(z) =
// 0.5 (1 + erf(z / sqrt 2)).  erf comes from Abramowitz & Stegun, Handbook of
// Mathematical Functions (1964), formula 7.1.26 (Hastings' rational
// approximation, |error| <= 1.5e-7): for x >= 0,
//   1 - erf(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
//   t = 1 / (1 + p x).
// With x = |z| / sqrt 2 and E = 0.5 (1 - erf(x)), Phi(z) = 1 - E for z >= 0
// and E for z < 0.  The constants below fold the 1/sqrt 2, the 0.5 and the
// natural-to-base-2 exponent into the coefficients, leaving one reciprocal,
// one exp2 and ten FMA-class operations.
__device__ __forceinline__ float gelu_erf(float z) {
    constexpr float kP = 0.3275911f * 0.70710678118654752f;   // p / sqrt 2
    constexpr float kE = -0.5f * 1.4426950408889634f;          // -x^2 log2(e) with x^2 = z^2 / 2
    const float t = __builtin_amdgcn_rcpf(fmaf(kP, fabsf(z), 1.0f));
    float q = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
    q = fmaf(q, t, 0.5f * 1.421413741f);
    q = fmaf(q, t, 0.5f * -0.284496736f);
    q = fmaf(q, t, 0.5f * 0.254829592f);
    const float ex = __builtin_amdgcn_exp2f((z * kE) * z);
    const float ze = z * (q * t) * ex;  // z * 0.5 (1 - erf(|z| / sqrt 2))
    return z >= 0.0f ? z - ze : ze;
}

}  // namespace wk
