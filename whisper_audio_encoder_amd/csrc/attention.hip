// Non-causal flash attention, head_dim 64, for gfx950.
//
// Computes, per (batch, head), O = softmax(Q K^T / 8) V over every key (whisper
// 0.9.0 API page, kernels.nu: the encoder attention is non-causal and its
// scores are q.k / sqrt(hd); the CKE page: the full 1500 x 1500 square, no
// mask, no RoPE).  The fused online-softmax form follows the idea the whisper
// README's performance notes give for its encoder kernel (one pass, the K/V
// stream amortised over many queries); the layout below is our own.
//
// One 256-thread workgroup takes 128 queries of one (b, h); each wave64 owns
// 32 of them.  Key tiles of 64 keys stream through LDS (double buffered):
// K as [key][64] and V^T as [dim][key], both in 16-byte chunks XOR-swizzled
// by row.  Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_f16, so a
// lane holds 32 scores of ONE query: the row max and row sum are in-lane
// reductions plus one exchange with lane ^ 32.  The probabilities are then
// already laid out as the B operand of O^T += V^T P^T; the order in which a
// lane holds its keys (4 consecutive keys, skip 4) is matched by storing
// each 16-key group of V^T in LDS in that same order.
//
// q arrives multiplied by log2(e) / 8, so the softmax is evaluated with
// exp2 and no further scaling.  Keys at or beyond T (the last tile of a
// 1500-key window) get score -inf and zero V.
#include "common.h"
#include "kernels.h"

namespace wk {

namespace {

constexpr int QT = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per tile

__global__ void __launch_bounds__(256)
attn_kernel(const f16 *__restrict__ q, const f16 *__restrict__ k, const f16 *__restrict__ vt,
            f16 *__restrict__ ao, int T, int H, int ldvt) {
    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, l32 = lane & 31;
    const int64_t bh = int64_t(b) * H + h;
    const f16 *Q = q + bh * T * 64;
    const f16 *K = k + bh * T * 64;
    const f16 *VT = vt + bh * 64 * ldvt;

    __shared__ __attribute__((aligned(16))) f16 Ks[2][KT * 64];
    __shared__ __attribute__((aligned(16))) f16 Vs[2][64 * KT];

    // Q^T fragments (B operand): lane supplies query l32, dims 16 kk + 8 hh .. +7.
    const int qrow = qt * QT + wave * 32 + l32;
    f16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        if (qrow < T)
            qf[kk] = *reinterpret_cast<const f16x8 *>(Q + int64_t(qrow) * 64 + kk * 16 + hh * 8);
        else
            qf[kk] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }

    // Tile staging: thread moves 16-byte chunk (tid & 7) of rows (tid >> 3) and (tid >> 3) + 32.
    const int ck = tid & 7;
    uint4 rk[2], rv[2];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = (tid >> 3) + 32 * i;
            const int key = kt * KT + r;
            rk[i] = key < T ? *reinterpret_cast<const uint4 *>(K + int64_t(key) * 64 + ck * 8) : make_uint4(0, 0, 0, 0);
            const int k0 = kt * KT + ck * 8;  // first key of this V^T chunk (row r = dim)
            uint4 v = make_uint4(0, 0, 0, 0);
            if (k0 < T) {
                v = *reinterpret_cast<const uint4 *>(VT + int64_t(r) * ldvt + k0);
                if (k0 + 8 > T) {
                    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (k0 + e >= T) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                    v = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
            rv[i] = v;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = (tid >> 3) + 32 * i;
            *reinterpret_cast<uint4 *>(&Ks[buf][r * 64 + ((ck ^ (r & 7)) << 3)]) = rk[i];
            // V^T chunk ck holds keys 8 ck .. 8 ck + 7 of 16-key group g = ck >> 1.
            // LDS chunk 2g + s holds, for lane half s, keys 16g + 4s + {0..3}
            // then 16g + 8 + 4s + {0..3}.
            const int lc0 = (ck >> 1) * 2, half = (ck & 1) * 4;
            *reinterpret_cast<uint2 *>(&Vs[buf][r * 64 + ((lc0 ^ (r & 7)) << 3) + half]) = make_uint2(rv[i].x, rv[i].y);
            *reinterpret_cast<uint2 *>(&Vs[buf][r * 64 + (((lc0 + 1) ^ (r & 7)) << 3) + half]) = make_uint2(rv[i].z, rv[i].w);
        }
    };

    f32x16 o[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        o[0][r] = 0.f;
        o[1][r] = 0.f;
    }
    float mrow = -INFINITY, lsum = 0.f;

    const int nkt = (T + KT - 1) / KT;
    gload(0);
    sstore(0);
    __syncthreads();
    const int fsw = lane & 7;
    for (int kt = 0; kt < nkt; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nkt) gload(kt + 1);

        // S^T tiles: rows = keys kt2*32 + 8 (r >> 2) + 4 hh + (r & 3), column = query l32.
        f32x16 s[2];
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt2][r] = 0.f;
            const f16 *kr = &Ks[cur][(kt2 * 32 + l32) * 64];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const f16x8 a = *reinterpret_cast<const f16x8 *>(kr + (((kk * 2 + hh) ^ fsw) << 3));
                s[kt2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[kk], s[kt2], 0, 0, 0);
            }
        }
        if ((kt + 1) * KT > T) {
#pragma unroll
            for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * KT + kt2 * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= T) s[kt2][r] = -INFINITY;
                }
        }

        float mx = s[0][0];
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt2][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrow, mx);
        const float alpha = exp2f(mrow - mnew);
        mrow = mnew;
        float ps = 0.f;
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = exp2f(s[kt2][r] - mnew);
                s[kt2][r] = e;
                ps += e;
            }
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            o[0][r] *= alpha;
            o[1][r] *= alpha;
        }

        // O^T[dim][query] += V^T[dim][keys] P^T[keys][query], 16 keys per MFMA.
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int kt2 = s4 >> 1, sg = s4 & 1;
            f16x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[i] = (f16)s[kt2][8 * sg + i];
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) {
                const int dim = ht * 32 + l32;
                const f16x8 va = *reinterpret_cast<const f16x8 *>(&Vs[cur][dim * 64 + (((2 * s4 + hh) ^ fsw) << 3)]);
                o[ht] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb, o[ht], 0, 0, 0);
            }
        }

        if (kt + 1 < nkt) sstore(cur ^ 1);
        __syncthreads();
    }

    lsum += __shfl_xor(lsum, 32);
    if (qrow < T) {
        const float inv = 1.0f / lsum;
        f16 *dst = ao + (int64_t(b) * T + qrow) * (int64_t(H) * 64) + h * 64;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dim = ht * 32 + 8 * g + 4 * hh;
                f16x4 w;
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (f16)(o[ht][4 * g + r] * inv);
                *reinterpret_cast<f16x4 *>(dst + dim) = w;
            }
    }
}

}  // namespace

const char *attention_check(int batch, int n_head, int T, int ldvt) {
    if (batch < 0 || n_head <= 0 || T <= 0) return "attention: need batch >= 0, n_head > 0, T > 0";
    if (ldvt < T || ldvt % 8) return "attention: ldvt must be >= T and a multiple of 8";
    if (n_head > 65535 || batch > 65535) return "attention: batch and n_head must be < 65536";
    return nullptr;
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *vt, uint16_t *ao,
                            int batch, int n_head, int T, int ldvt, hipStream_t s) {
    if (batch == 0) return hipSuccess;
    const dim3 grid((T + QT - 1) / QT, n_head, batch), block(256);
    attn_kernel<<<grid, block, 0, s>>>(reinterpret_cast<const f16 *>(q), reinterpret_cast<const f16 *>(k),
                                       reinterpret_cast<const f16 *>(vt), reinterpret_cast<f16 *>(ao), T, n_head,
                                       ldvt);
    return hipGetLastError();
}

}  // namespace wk
