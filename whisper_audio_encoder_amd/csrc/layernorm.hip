// LayerNorm (with bias) and mel ingest, for gfx950.  Both are bound by HBM
// bandwidth: each row is read once and written once with 16-byte loads.
//
// LayerNorm (whisper 0.9.0 API page, kernels.nu: it subtracts the mean and
// has a bias, unlike RMSNorm): one wave64 per row at a time, the row held
// in registers (float4 per lane per 256 columns), two passes over those
// registers for the mean and the population variance, wave reductions by
// lane exchange.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace wk {

namespace {

// Sum over the 64 lanes with DPP moves (no LDS round trips): within each
// quad, then 8- and 16-lane rows (mirrors), then rows 0+1 -> 1 and 2+3 -> 3
// (broadcast of lane 15), then 0..3 -> 3 (broadcast of lane 31); lane 63
// ends with the total, which every lane reads.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false);
    return v + __int_as_float(moved);
}

__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xf>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xf>(v);  // row_mirror
    v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// A 256-lane workgroup holds four waves; wave w of the grid takes rows w,
// w + n_waves, ... and issues the next row's loads before it reduces the
// current one, so a wave always has a row in flight (measured at 24000 x
// 1280: 32.6 -> 29.9 us against one 64-lane workgroup per row, the same
// bits; at 24000 x 768 unchanged).
template <int NV, bool OUT32>
__global__ void __launch_bounds__(256)
ln_kernel(const float *__restrict__ x, const float *__restrict__ g, const float *__restrict__ bta,
          void *__restrict__ y, int rows, int d, float eps) {
    const int lane = threadIdx.x & 63;
    const int nwaves = gridDim.x * 4;
    // (readfirstlane: the row is uniform across the wave, so the buffer
    // descriptors below stay in scalar registers)
    int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int nv = d >> 2;
    float4 v[NV], vn[NV], gg[NV], bb[NV];
    // Buffer loads over the one row (a row past the last one has an empty
    // range): columns past d read zero without a branch, so the compiler's
    // wait before the current row's use counts the next row's loads exactly
    // instead of waiting for them too.
    auto load = [&](int r, float4 (&dst)[NV]) {
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(x) + int64_t(r < rows ? r : 0) * d, 0, r < rows ? d * 4 : 0, 0x00020000);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const f32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rx, uint32_t(lane + 64 * j) * 16u, 0, 0);
            dst[j] = make_float4(t[0], t[1], t[2], t[3]);
        }
    };
    // the gains and biases once per wave, before the rows (no load inside
    // the row loop but the next row's)
    {
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(g), 0, d * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(bta), 0, d * 4, 0x00020000);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const f32x4 tg = __builtin_amdgcn_raw_buffer_load_b128(rg, uint32_t(lane + 64 * j) * 16u, 0, 0);
            const f32x4 tb = __builtin_amdgcn_raw_buffer_load_b128(rb, uint32_t(lane + 64 * j) * 16u, 0, 0);
            gg[j] = make_float4(tg[0], tg[1], tg[2], tg[3]);
            bb[j] = make_float4(tb[0], tb[1], tb[2], tb[3]);
        }
    }
    load(row, v);
    for (; row < rows; row += nwaves) {
        load(row + nwaves, vn);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
        const float mean = wave_sum(s) / float(d);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = lane + 64 * j;
            if (i < nv) {
                const float a = v[j].x - mean, b = v[j].y - mean, c = v[j].z - mean, e = v[j].w - mean;
                ss += (a * a + b * b) + (c * c + e * e);
            }
        }
        const float rstd = 1.0f / sqrtf(wave_sum(ss) / float(d) + eps);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = lane + 64 * j;
            if (i < nv) {
                const float o0 = (v[j].x - mean) * rstd * gg[j].x + bb[j].x;
                const float o1 = (v[j].y - mean) * rstd * gg[j].y + bb[j].y;
                const float o2 = (v[j].z - mean) * rstd * gg[j].z + bb[j].z;
                const float o3 = (v[j].w - mean) * rstd * gg[j].w + bb[j].w;
                if constexpr (OUT32) {
                    reinterpret_cast<float4 *>(static_cast<float *>(y) + int64_t(row) * d)[i] = make_float4(o0, o1, o2, o3);
                } else {
                    f16x4 w = {(f16)o0, (f16)o1, (f16)o2, (f16)o3};
                    reinterpret_cast<f16x4 *>(static_cast<f16 *>(y) + int64_t(row) * d)[i] = w;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = vn[j];
    }
}

template <int NV>
hipError_t ln_dispatch(const float *x, const float *g, const float *b, void *y, int rows, int d, float eps,
                       bool out_f32, hipStream_t s) {
    // 4096 workgroups (16 per CU) of four waves, or fewer for short inputs
    // (measured: 2048 and 4096 equal, 1024 3% and 512 10% slower at 24000 x 1280)
    const dim3 grid(unsigned(std::min((rows + 3) / 4, 4096))), block(256);
    if (out_f32)
        ln_kernel<NV, true><<<grid, block, 0, s>>>(x, g, b, y, rows, d, eps);
    else
        ln_kernel<NV, false><<<grid, block, 0, s>>>(x, g, b, y, rows, d, eps);
    return hipGetLastError();
}

// melp[b][r][c] = r in [1, F] ? fp16(mel[b][r-1][c]) : 0, four values per
// thread; then rows 0 and F+1 of c1[b] are cleared.
__global__ void __launch_bounds__(256)
ingest_kernel(const float *__restrict__ mel, f16 *__restrict__ melp, f16 *__restrict__ c1, int B, int F, int nm,
              int d) {
    const int64_t n1 = int64_t(B) * (F + 2) * (nm >> 2);
    const int64_t n2 = int64_t(B) * 2 * (d >> 2);
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n1 + n2; i += stride) {
        if (i < n1) {
            const int64_t per_item = int64_t(F + 2) * (nm >> 2);
            const int64_t b = i / per_item;
            const int64_t rem = i - b * per_item;
            const int r = int(rem / (nm >> 2));
            const int c4 = int(rem - int64_t(r) * (nm >> 2));
            f16x4 w = {0, 0, 0, 0};
            if (r >= 1 && r <= F) {
                const float4 v = reinterpret_cast<const float4 *>(mel + (b * F + (r - 1)) * nm)[c4];
                w = f16x4{(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w};
            }
            reinterpret_cast<f16x4 *>(melp + (b * (F + 2) + r) * nm)[c4] = w;
        } else {
            const int64_t j = i - n1;
            const int64_t per_item = 2 * (d >> 2);
            const int64_t b = j / per_item;
            const int64_t rem = j - b * per_item;
            const int which = int(rem / (d >> 2));
            const int c4 = int(rem - int64_t(which) * (d >> 2));
            const int64_t row = b * (F + 2) + (which ? F + 1 : 0);
            reinterpret_cast<f16x4 *>(c1 + row * d)[c4] = f16x4{0, 0, 0, 0};
        }
    }
}

// y = fp16(x), round to nearest even, four values per thread (n4 groups).
__global__ void __launch_bounds__(256)
to_f16_kernel(const float4 *__restrict__ x, f16x4 *__restrict__ y, int64_t n4) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 v = x[i];
        y[i] = f16x4{(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w};
    }
}

}  // namespace

const char *layernorm_check(int rows, int d) {
    if (rows < 0) return "layernorm: rows < 0";
    if (d <= 0 || d % 4 || d > 2048) return "layernorm: need 0 < d <= 2048 and d % 4 == 0";
    return nullptr;
}

hipError_t launch_layernorm(const float *x, const float *g, const float *b, void *y, int rows, int d, float eps,
                            bool out_f32, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int nv = (d / 4 + 63) / 64;
    switch (nv) {
        case 1: return ln_dispatch<1>(x, g, b, y, rows, d, eps, out_f32, s);
        case 2: return ln_dispatch<2>(x, g, b, y, rows, d, eps, out_f32, s);
        case 3: return ln_dispatch<3>(x, g, b, y, rows, d, eps, out_f32, s);
        case 4: return ln_dispatch<4>(x, g, b, y, rows, d, eps, out_f32, s);
        case 5: return ln_dispatch<5>(x, g, b, y, rows, d, eps, out_f32, s);
        case 6: return ln_dispatch<6>(x, g, b, y, rows, d, eps, out_f32, s);
        case 7: return ln_dispatch<7>(x, g, b, y, rows, d, eps, out_f32, s);
        case 8: return ln_dispatch<8>(x, g, b, y, rows, d, eps, out_f32, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ingest(const float *mel, uint16_t *melp, uint16_t *c1, int B, int F, int nm, int d, hipStream_t s) {
    if (B == 0) return hipSuccess;
    const int64_t n = int64_t(B) * (F + 2) * (nm / 4) + int64_t(B) * 2 * (d / 4);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    ingest_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(mel, reinterpret_cast<f16 *>(melp),
                                                             reinterpret_cast<f16 *>(c1), B, F, nm, d);
    return hipGetLastError();
}

hipError_t launch_to_f16(const float *x, uint16_t *y, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (n % 4) return hipErrorInvalidValue;
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    to_f16_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(reinterpret_cast<const float4 *>(x),
                                                             reinterpret_cast<f16x4 *>(y), n / 4);
    return hipGetLastError();
}

}  // namespace wk
