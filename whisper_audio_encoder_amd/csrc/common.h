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
// Mathematical Functions (1964), formula 7.1.28 (|error| <= 3e-7): for x >= 0,
//   1 - erf(x) = (1 + a1 x + a2 x^2 + a3 x^3 + a4 x^4 + a5 x^5 + a6 x^6)^-16.
// With x = |z| / sqrt 2 and r = 0.5 (1 - erf(x)), Phi(z) = 1 - r for z >= 0
// and r for z < 0, so in both cases gelu(z) = max(z, 0) - |z| r.  The
// coefficients below are a_k 2^(-k/2) (the 1/sqrt 2 folded in) times
// 2^(1/16) (so the 16th power carries the 0.5), leaving six FMAs, four
// squarings, one reciprocal and one FMA.  In fp32 the result is within
// 7.1e-7 of the exact GELU everywhere (checked on a dense grid over
// [-12, 12]); for large |z| the 16th power overflows to +inf, r to 0 and the
// result to max(z, 0), as it should.
__device__ __forceinline__ float gelu_erf(float z) {
    const float u = fabsf(z);
    float q = fmaf(5.621299806e-06f, u, 5.105520904e-05f);
    q = fmaf(q, u, 3.968613601e-05f);
    q = fmaf(q, u, 3.422739217e-03f);
    q = fmaf(q, u, 2.207699791e-02f);
    q = fmaf(q, u, 5.207516253e-02f);
    q = fmaf(q, u, 1.044273734e+00f);
    q *= q;
    q *= q;
    q *= q;
    q *= q;
    const float r = __builtin_amdgcn_rcpf(q);
    // max(z, 0) as one instruction: fmaxf would first quiet a signalling NaN
    // with an extra max.  A NaN z still yields NaN through -u.
    float pos;
    asm("v_max_f32_e32 %0, 0, %1" : "=v"(pos) : "v"(z));
    return fmaf(-u, r, pos);
}

}  // namespace wk
