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
// 0.5 (1 + erf(z / sqrt 2)).  With Q(u) = Phi(-u), the upper normal tail,
// Phi(z) = 1 - Q(|z|) for z >= 0 and Q(|z|) for z < 0, so in both cases
// gelu(z) = max(z, 0) - |z| Q(|z|).  Q is evaluated as 2^p(u), p a degree-5
// polynomial fitted to log2 Q on [0, 6] so as to minimise the largest error
// of u Q(u) (tests/gelu_tail_fit.py derives the coefficients, and
// tests/test_gelu_constants.py checks the ones below against the exact GELU
// in the same fp32 arithmetic): five FMAs, one exp2, one max and one FMA.
// In fp32 the result
// is within 4.7e-7 of the exact GELU everywhere (dense grid over [-12, 12]);
// p decreases for all u >= 0, so past the fitted range the tail term keeps
// shrinking (< 5e-9 beyond u = 6) and exp2 underflows to 0 for large |z|,
// leaving max(z, 0).
__device__ __forceinline__ float gelu_erf(float z) {
    const float u = fabsf(z);
    float p = fmaf(-4.733079986e-4f, u, 7.084549870e-3f);
    p = fmaf(p, u, -5.182737112e-2f);
    p = fmaf(p, u, -4.599924386e-1f);
    p = fmaf(p, u, -1.150787830e+0f);
    p = fmaf(p, u, -1.000037670e+0f);
    const float r = __builtin_amdgcn_exp2f(p);
    // max(z, 0) as one instruction: fmaxf would first quiet a signalling NaN
    // with an extra max.  A NaN z still yields NaN through -u.
    float pos;
    asm("v_max_f32_e32 %0, 0, %1" : "=v"(pos) : "v"(z));
    return fmaf(-u, r, pos);
}

}  // namespace wk
