// Decode-step cross-attention over the cached encoder K/V, for gfx950.
//
// A decoder step has one query per sequence (a few with beams), and every
// decoder layer attends over the n_ctx (1500) encoder positions through the
// K/V that wenc_prepare_cross cached once per clip (whisper 0.9.0 API page,
// wh_prepare_cross; model.nu: x_wk, x_wv).  Per (batch item, head h, query):
//   out = softmax_u(q . xk[u] / sqrt(64)) xv[u]
// over columns [64h, 64h + 64) (kernels.nu: scores q.k / sqrt(hd)).  With one
// query the encoder's kernel, which amortises each key tile over 128 queries,
// would leave the chip idle; the whisper README ("Performance and memory")
// describes the remedy its one-query kernel uses: split the keys across
// workgroups and merge the partial softmaxes.  The layout below is our own.
//
// Two passes (the default) or one, chosen per launch (xattn_one_pass).
// Pass 1 (xattn_partial): a workgroup takes 64 keys per wave of one (b, h);
// K and V rows are read 8 lanes to a row (16 bytes a lane), the partial dot
// products of a key's 8 lanes (fp16 pairs accumulated in fp32) are summed by
// a reduce-scatter that leaves one key's score per lane, a wave takes its
// maximum and exp2 sum, then accumulates P.V with the same 8 lanes per value
// row; the waves merge through LDS and write the workgroup's (max, sum,
// o[64]) per query.  Pass 2
// (xattn_merge): one wave per (b, h) rescales the partials to a common
// maximum and sums them in key order, so the result does not depend on
// scheduling.  One pass (xattn_whole): a workgroup per (b, h) walks all its
// keys, 64 per wave at a time, with an online softmax, and writes out.  The
// work is bound by reading K and V once (HBM).
#include "common.h"
#include "kernels.h"

namespace wk {

namespace {

// Waves per workgroup of pass 1 (each takes 64 keys) for NQ query rows.
// Measured at 16 windows x 1500 keys x 20 heads: 8 waves against 4 is 5%
// faster per layer (both passes) for one query and 9% for four, and 7% slower
// for eight, whose larger per-lane state makes the wider workgroup's waves
// wait longer.  The saving is the merge's, which reads half as many partials;
// pass 1 alone is a few percent slower with 8 waves.
constexpr int xnw(int nq) { return nq <= 4 ? 8 : 4; }
constexpr int xkc(int nq) { return 64 * xnw(nq); }  // keys per workgroup of pass 1
constexpr int XNW_MIN = 4;  // the fewest keys per workgroup over every NQ: 64 XNW_MIN
constexpr int XPART = 68;  // floats per partial: max, sum, o[64], 2 pad (16-byte rows)
constexpr float LOG2E_8 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_add(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Buffer descriptor over one window's K or V rows: offsets at or past the
// window's T rows read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t xrsrc(const f16 *x, int b, int T, int64_t d) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<f16 *>(x) + int64_t(b) * T * d, 0,
                                             int(uint32_t(T) * uint32_t(d) * 2u), 0x00020000);
}

// K and V rows are both read 8 lanes to a row: in load it, lane (r8 = lane
// >> 3, dq = lane & 7) holds dimensions 8 dq .. +7 of key key0 + 8 it + r8,
// so one instruction covers 8 whole 128-byte rows.  Buffer loads: a key at
// or past T has an offset past the range and reads zero.  All are issued
// before the scores, K first.
__device__ __forceinline__ void xload(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int key0, int T,
                                      int64_t d, int h, int dq, int r8, f16x8 (&kv)[8], f16x8 (&vv)[8]) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int uu = key0 + 8 * it + r8;
        const uint32_t off = uu < T ? uint32_t((int64_t(uu) * d + h * 64 + 8 * dq) * 2) : 0x80000000u;
        kv[it] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int uu = key0 + 8 * it + r8;
        const uint32_t off = uu < T ? uint32_t((int64_t(uu) * d + h * 64 + 8 * dq) * 2) : 0x80000000u;
        vv[it] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
}

// Scores (base 2, scaled by log2(e)/8) of the loaded keys: each lane's
// partial dot product over its 8 dimensions, then a reduce-scatter over the
// 8 lanes of a row (exchanging 4, 2, 1 partials with lanes dq ^ 4, ^ 2, ^ 1),
// after which lane (r8, dq) holds the whole score of key u = key0 + 8 dq +
// r8 (-inf for u >= T).
template <int NQ>
__device__ __forceinline__ void xscores(const f16x8 (&kv)[8], const f16x2 (&qs)[NQ][32], int u, int T, int dq,
                                        float (&s)[NQ]) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        float v8[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc = __builtin_amdgcn_fdot2(f16x2{kv[it][2 * t], kv[it][2 * t + 1]}, qs[i][4 * dq + t], acc, false);
            v8[it] = acc;
        }
        float v4[4], v2[2];
        const bool b4 = dq & 4, b2 = dq & 2, b1 = dq & 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = (b4 ? v8[j + 4] : v8[j]) + __shfl_xor(b4 ? v8[j] : v8[j + 4], 4);
#pragma unroll
        for (int j = 0; j < 2; ++j) v2[j] = (b2 ? v4[j + 2] : v4[j]) + __shfl_xor(b2 ? v4[j] : v4[j + 2], 2);
        const float full = (b1 ? v2[1] : v2[0]) + __shfl_xor(b1 ? v2[0] : v2[1], 1);
        s[i] = u < T ? full * LOG2E_8 : -INFINITY;
    }
}

// oa += P.V over the loaded rows: lane (r8, dq) takes the probabilities of
// keys 8 it + r8 from the wave's LDS row ps (written by the same wave: LDS
// operations of a wave complete in order) against its 8 dimensions of them.
template <int NQ>
__device__ __forceinline__ void xpv(const f16x8 (&vv)[8], const float (&ps)[NQ][64], int r8, float (&oa)[NQ][8]) {
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const float p = ps[i][8 * it + r8];
#pragma unroll
            for (int e = 0; e < 8; ++e) oa[i][e] = fmaf(p, float(vv[it][e]), oa[i][e]);
        }
}

// Sum over the 8 lanes that share a dimension group (lane bits 3..5); lanes
// with r8 == 0 then write the wave's o[64] per query.
template <int NQ>
__device__ __forceinline__ void xreduce_store(float (&oa)[NQ][8], float (&wo)[NQ][64], int r8, int dq) {
#pragma unroll
    for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            oa[i][e] += __shfl_xor(oa[i][e], 8);
            oa[i][e] += __shfl_xor(oa[i][e], 16);
            oa[i][e] += __shfl_xor(oa[i][e], 32);
        }
    if (r8 == 0) {
#pragma unroll
        for (int i = 0; i < NQ; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) wo[i][8 * dq + e] = oa[i][e];
    }
}

// The queries of (b, h) as fp16 pairs in LDS.
template <int NQ, int NT>
__device__ __forceinline__ void xload_q(const f16 *q, f16x2 (&qs)[NQ][32], int b, int h, int64_t d, int tid) {
    for (int i = tid; i < NQ * 32; i += NT) {
        const int qi = i / 32, e2 = i % 32;
        qs[qi][e2] = *reinterpret_cast<const f16x2 *>(q + (int64_t(b) * NQ + qi) * d + h * 64 + 2 * e2);
    }
}

// Pass 1's work for one wave: the 64 keys key0 .. key0 + 63 of (b, h) give
// the wave's maximum, exp2 sum and o[64] per query, written to its rows of
// wm, wl and wo (a wave whose keys all lie at or past T has maximum -inf,
// sum 0 and o 0).
template <int NQ, int XNW>
__device__ __forceinline__ void xwave_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int key0, int T,
                                           int64_t d, int h, int lane, int wave, const f16x2 (&qs)[NQ][32],
                                           float (&ps)[XNW][NQ][64], float (&wm)[XNW][NQ], float (&wl)[XNW][NQ],
                                           float (&wo)[XNW][NQ][64]) {
    const int dq = lane & 7, r8 = lane >> 3;
    f16x8 kv[8], vv[8];
    xload(rk, rv, key0, T, d, h, dq, r8, kv, vv);
    const int u = key0 + 8 * dq + r8;
    float s[NQ];
    xscores<NQ>(kv, qs, u, T, dq, s);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const float m = wave_max(s[i]);  // -inf only when every key of the wave is past T
        const float p = u < T ? __builtin_amdgcn_exp2f(s[i] - m) : 0.f;
        const float l = wave_add(p);
        ps[wave][i][8 * dq + r8] = p;
        if (lane == 0) {
            wm[wave][i] = m;
            wl[wave][i] = l;
        }
    }
    float oa[NQ][8];
#pragma unroll
    for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) oa[i][e] = 0.f;
    xpv<NQ>(vv, ps[wave], r8, oa);
    xreduce_store<NQ>(oa, wo[wave], r8, dq);
}

// A workgroup's partial for query i, column e: its waves at a common maximum,
// in wave order (a wave with maximum -inf has weight 0).
template <int NQ, int XNW>
__device__ __forceinline__ void xmerge_waves(const float (&wm)[XNW][NQ], const float (&wl)[XNW][NQ],
                                             const float (&wo)[XNW][NQ][64], int i, int e, float &M, float &L,
                                             float &O) {
    M = wm[0][i];
#pragma unroll
    for (int w = 1; w < XNW; ++w) M = fmaxf(M, wm[w][i]);
    L = 0.f;
    O = 0.f;
#pragma unroll
    for (int w = 0; w < XNW; ++w) {
        const float sc = __builtin_amdgcn_exp2f(wm[w][i] - M);
        L = fmaf(sc, wl[w][i], L);
        O = fmaf(sc, wo[w][i][e], O);
    }
}

// Pass 2's merge of nc chunk partials (max m(c), sum l(c), column o(c)) in
// chunk order: the output value sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c.
template <class Fm, class Fl, class Fo>
__device__ __forceinline__ float xmerge_chunks(int nc, Fm m, Fl l, Fo o) {
    float M = m(0);
    for (int c = 1; c < nc; ++c) M = fmaxf(M, m(c));
    float L = 0.f, O = 0.f;
    for (int c = 0; c < nc; ++c) {
        const float sc = __builtin_amdgcn_exp2f(m(c) - M);
        L = fmaf(sc, l(c), L);
        O = fmaf(sc, o(c), O);
    }
    return O / L;
}

template <int NQ, int XNW = xnw(NQ)>
__global__ void __launch_bounds__(64 * XNW)
xattn_partial(const f16 *__restrict__ q, const f16 *__restrict__ xk, const f16 *__restrict__ xv,
              float *__restrict__ part, int T, int H, int nc) {
    const int wg = blockIdx.x;
    const int c = wg % nc, bh = wg / nc;
    const int h = bh % H, b = bh / H;
    const int64_t d = int64_t(H) * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    __shared__ f16x2 qs[NQ][32];      // the queries of (b, h), fp16 pairs
    __shared__ float ps[XNW][NQ][64];  // probabilities, by wave and key
    __shared__ float wm[XNW][NQ], wl[XNW][NQ];
    __shared__ float wo[XNW][NQ][64];

    xload_q<NQ, 64 * XNW>(q, qs, b, h, d, tid);
    __syncthreads();

    xwave_tile<NQ, XNW>(xrsrc(xk, b, T, d), xrsrc(xv, b, T, d), c * (64 * XNW) + wave * 64, T, d, h, lane, wave, qs,
                        ps, wm, wl, wo);
    __syncthreads();

    // the workgroup's partial per query
    for (int idx = tid; idx < NQ * 64; idx += 64 * XNW) {
        const int i = idx / 64, e = idx % 64;
        float M, L, O;
        xmerge_waves<NQ, XNW>(wm, wl, wo, i, e, M, L, O);
        float *pp = part + ((int64_t(bh) * nc + c) * NQ + i) * XPART;
        pp[2 + e] = O;
        if (e == 0) {
            pp[0] = M;
            pp[1] = L;
        }
    }
}

// One pass, for batches whose (b, h) pairs about fill the compute units: a
// workgroup takes every key of one (b, h) and runs both passes' arithmetic
// in their order, so its output has the same bits as the two launches.  In
// round c its waves take the 64-key tiles of key chunk c (64 XNW keys) as
// pass 1 does and merge them into the chunk's (max, sum, o[64]), kept in
// LDS; after the last round the chunks merge as pass 2 does.  No partials
// leave the chip and no second launch follows.  nc <= XNC_MAX.
constexpr int XNC_MAX = 8;

template <int NQ, int XNW = xnw(NQ)>
__global__ void __launch_bounds__(64 * XNW)
xattn_whole(const f16 *__restrict__ q, const f16 *__restrict__ xk, const f16 *__restrict__ xv,
            f16 *__restrict__ out, int T, int H, int nc) {
    const int bh = blockIdx.x;
    const int h = bh % H, b = bh / H;
    const int64_t d = int64_t(H) * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    __shared__ f16x2 qs[NQ][32];
    __shared__ float ps[XNW][NQ][64];
    __shared__ float wm[XNW][NQ], wl[XNW][NQ];
    __shared__ float wo[XNW][NQ][64];
    __shared__ float cm[XNC_MAX][NQ], cl[XNC_MAX][NQ];
    __shared__ float co[XNC_MAX][NQ][64];

    xload_q<NQ, 64 * XNW>(q, qs, b, h, d, tid);
    __syncthreads();

    const __amdgpu_buffer_rsrc_t rk = xrsrc(xk, b, T, d), rv = xrsrc(xv, b, T, d);
    for (int c = 0; c < nc; ++c) {
        xwave_tile<NQ, XNW>(rk, rv, c * (64 * XNW) + wave * 64, T, d, h, lane, wave, qs, ps, wm, wl, wo);
        __syncthreads();
        for (int idx = tid; idx < NQ * 64; idx += 64 * XNW) {
            const int i = idx / 64, e = idx % 64;
            float M, L, O;
            xmerge_waves<NQ, XNW>(wm, wl, wo, i, e, M, L, O);
            co[c][i][e] = O;
            if (e == 0) {
                cm[c][i] = M;
                cl[c][i] = L;
            }
        }
        __syncthreads();  // the next round rewrites wm, wl and wo
    }

    for (int idx = tid; idx < NQ * 64; idx += 64 * XNW) {
        const int i = idx / 64, e = idx % 64;
        out[(int64_t(b) * NQ + i) * d + h * 64 + e] = f16(xmerge_chunks(
            nc, [&](int c) { return cm[c][i]; }, [&](int c) { return cl[c][i]; }, [&](int c) { return co[c][i][e]; }));
    }
}

// One wave per (b, h): out = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c,
// in key-chunk order.
template <int NQ>
__global__ void __launch_bounds__(64)
xattn_merge(const float *__restrict__ part, f16 *__restrict__ out, int H, int nc) {
    const int bh = blockIdx.x, e = threadIdx.x;
    const int h = bh % H, b = bh / H;
    const int64_t d = int64_t(H) * 64;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const float *p0 = part + (int64_t(bh) * nc * NQ + i) * XPART;
        const int64_t cs = int64_t(NQ) * XPART;  // floats from one chunk's partial to the next
        out[(int64_t(b) * NQ + i) * d + h * 64 + e] = f16(xmerge_chunks(
            nc, [&](int c) { return p0[c * cs]; }, [&](int c) { return p0[c * cs + 1]; },
            [&](int c) { return p0[c * cs + 2 + e]; }));
    }
}

// One pass or two.  The one pass takes a (b, h) in rounds, one key chunk
// each, so it pays when the pairs nearly fill the compute units once: with
// fewer, too few units pull from memory; with more, some units hold two
// workgroups and finish last, while the two-pass split balances them.
// Measured per layer at 1500 keys over 80 to 320 pairs on 256 units (4, 8,
// 12, 16 windows x 20 heads; 16 x 12): up to 4 query rows the one pass wins
// at 0.75 and 0.94 pairs per unit (-5% to -8%) and loses at 0.31, 0.63 and
// 1.25.  With 5 to 8 rows (256-key chunks, six rounds of two barriers each)
// it loses everywhere.  The bits are the same either way.
bool xattn_one_pass(int64_t pairs, int nq, long cus) {
    const double r = double(pairs) / double(cus);
    return nq <= 4 && r >= 0.7 && r <= 1.0;
}

template <int NQ>
hipError_t xattn_dispatch(const f16 *q, const f16 *xk, const f16 *xv, f16 *out, float *part, int B, int H, int T,
                          hipStream_t s) {
    const int nc = (T + xkc(NQ) - 1) / xkc(NQ);
    if (nc <= XNC_MAX && xattn_one_pass(int64_t(B) * H, NQ, cu_count())) {
        xattn_whole<NQ><<<dim3(unsigned(B * H)), dim3(64 * xnw(NQ)), 0, s>>>(q, xk, xv, out, T, H, nc);
        return hipGetLastError();
    }
    xattn_partial<NQ><<<dim3(unsigned(B * H * nc)), dim3(64 * xnw(NQ)), 0, s>>>(q, xk, xv, part, T, H, nc);
    xattn_merge<NQ><<<dim3(unsigned(B * H)), dim3(64), 0, s>>>(part, out, H, nc);
    return hipGetLastError();
}

}  // namespace

size_t xattn_part_bytes(int batch, int n_head, int n_q, int T) {
    const size_t nc = size_t(T + xkc(n_q) - 1) / xkc(n_q);
    return size_t(batch) * n_head * nc * n_q * XPART * sizeof(float);
}

const char *xattn_check(int batch, int n_head, int n_q, int T) {
    if (batch < 0 || n_head <= 0) return "cross attention: need batch >= 0, n_head > 0";
    if (n_q < 1 || n_q > XATTN_MAX_Q) return "cross attention: n_q must be in [1, 8]";
    if (T < 1) return "cross attention: n_ctx must be >= 1";
    if (int64_t(T) * n_head * 64 * 2 >= (int64_t(1) << 31)) return "cross attention: a window's K or V exceeds 2 GiB";
    if (int64_t(batch) * n_head * ((T + 64 * XNW_MIN - 1) / (64 * XNW_MIN)) >= (int64_t(1) << 31))
        return "cross attention: grid too large";
    return nullptr;
}

hipError_t launch_xattn(const uint16_t *q, const uint16_t *xk, const uint16_t *xv, uint16_t *out, float *part,
                        int batch, int n_head, int n_q, int T, hipStream_t s) {
    if (batch == 0) return hipSuccess;
    const f16 *q16 = reinterpret_cast<const f16 *>(q), *k16 = reinterpret_cast<const f16 *>(xk),
              *v16 = reinterpret_cast<const f16 *>(xv);
    f16 *o16 = reinterpret_cast<f16 *>(out);
    switch (n_q) {
        case 1: return xattn_dispatch<1>(q16, k16, v16, o16, part, batch, n_head, T, s);
        case 2: return xattn_dispatch<2>(q16, k16, v16, o16, part, batch, n_head, T, s);
        case 3: return xattn_dispatch<3>(q16, k16, v16, o16, part, batch, n_head, T, s);
        case 4: return xattn_dispatch<4>(q16, k16, v16, o16, part, batch, n_head, T, s);
        case 5: return xattn_dispatch<5>(q16, k16, v16, o16, part, batch, n_head, T, s);
        case 6: return xattn_dispatch<6>(q16, k16, v16, o16, part, batch, n_head, T, s);
        case 7: return xattn_dispatch<7>(q16, k16, v16, o16, part, batch, n_head, T, s);
        case 8: return xattn_dispatch<8>(q16, k16, v16, o16, part, batch, n_head, T, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wk
