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

// Exact GELU, the error-function form: 0.5 z (1 + erf(z / sqrt 2)).
// erff is the ROCm device library's.
__device__ __forceinline__ float gelu_erf(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

}  // namespace wk
