// fp16 MFMA GEMM with fused epilogues, for gfx950.
//
//   acc[m][n] = sum_k A[m][k] * W[n][k]       (both operands K-contiguous)
//
// This one kernel carries every dense contraction of the encoder: the conv
// stem (conv1, conv2 as GEMMs over overlapping frame windows, whisper 0.9.0
// API page, model.nu: k=3, pad=1, strides 1 and 2), the fused q|k|v
// projection (k without bias, model.nu), out_proj and fc2 with the residual
// add, and fc1 with the erf GELU (kernels.nu).  Matrices are [out][in]
// (kernels.nu, wk_matvec: W[rows][cols]), so W rows are K-contiguous, which
// is exactly the operand layout v_mfma_f32_32x32x16_f16 reads per lane.
//
// Structure: a 256-thread workgroup (4 wave64s) owns a BM x BN output tile
// and walks K in steps of 64.  Each step is staged through LDS with 16-byte
// chunks XOR-swizzled by row (chunk c of row r lives at c ^ (r & 7)) so the
// 16-byte fragment reads of 8 consecutive rows hit distinct banks.  LDS is
// double buffered: the next K step's global loads are in flight while the
// current step's MFMAs run, and one barrier per step separates them.
// Workgroup ids are remapped so each XCD (ids are dealt round-robin over the
// 8 XCDs) receives a contiguous run of tiles, ordered in groups of 8 tile
// rows, so tiles sharing A rows or W rows share that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace wk {

namespace {

constexpr int BK = 64;

struct GemmP {
    const f16 *A;
    int64_t a_bs;
    DivU a_div;
    int lda;
    const f16 *W;
    int ldw;
    const float *bias;
    void *C;
    int64_t c_bs;
    DivU c_div;
    int c_off;
    int ldc;
    const float *pos;
    DivU pos_div;
    f16 *q, *k, *vt;
    DivU t_div;
    int H, ldvt, dmodel;
    float q_scale;
    int M, N, K;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ void tile_coords(int bid, int nwg, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int per = nwg >> 3, rem = nwg & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    const int lid = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    constexpr int GM = 8;
    const int group_size = GM * tiles_n;
    const int g = lid / group_size;
    const int first_m = g * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in = lid - g * group_size;
    tm = first_m + in % gm;
    tn = in / gm;
}

template <int EPI>
__device__ __forceinline__ void epi_store(const GemmP &p, int m, int n, float v) {
    if constexpr (EPI == WENC_EPI_GELU_F16) {
        const uint32_t bi = divu(m, p.c_div);
        const uint32_t r = m - bi * p.c_div.d;
        f16 *C = static_cast<f16 *>(p.C) + bi * p.c_bs + int64_t(r + p.c_off) * p.ldc + n;
        *C = (f16)gelu_erf(v + p.bias[n]);
    } else if constexpr (EPI == WENC_EPI_CONV2) {
        const uint32_t t = m - divu(m, p.pos_div) * p.pos_div.d;
        float *C = static_cast<float *>(p.C) + int64_t(m) * p.ldc + n;
        *C = gelu_erf(v + p.bias[n]) + p.pos[int64_t(t) * p.N + n];
    } else if constexpr (EPI == WENC_EPI_RESID) {
        float *C = static_cast<float *>(p.C) + int64_t(m) * p.ldc + n;
        *C += v + p.bias[n];
    }
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 2)))
gemm_kernel(const GemmP p) {
    constexpr int WAVES_N = BN / WN;
    static_assert((BM / WM) * (BN / WN) == 4, "4 waves per workgroup");
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int AL = BM * (BK / 8) / 256;
    constexpr int BL = BN * (BK / 8) / 256;
    __shared__ __attribute__((aligned(16))) f16 smem[2 * (BM + BN) * BK];
    f16 *As = smem;
    f16 *Bs = smem + 2 * BM * BK;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Global -> LDS staging: thread t moves 16-byte chunk (t & 7) of rows
    // (t >> 3) + 32 i.  The chunk's k offset is the same for every i.
    const int ck = tid & 7;
    const f16 *a_src[AL];
    bool a_ok[AL];
    int a_dst[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int m = m0 + r;
        a_ok[i] = m < p.M;
        const uint32_t mm = a_ok[i] ? m : 0;
        const uint32_t bi = divu(mm, p.a_div);
        a_src[i] = p.A + bi * p.a_bs + int64_t(mm - bi * p.a_div.d) * p.lda + ck * 8;
        a_dst[i] = r * BK + ((ck ^ (r & 7)) << 3);
    }
    const f16 *b_src[BL];
    bool b_ok[BL];
    int b_dst[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int n = n0 + r;
        b_ok[i] = n < p.N;
        b_src[i] = p.W + int64_t(b_ok[i] ? n : 0) * p.ldw + ck * 8;
        b_dst[i] = r * BK + ((ck ^ (r & 7)) << 3);
    }

    uint4 ra[AL], rb[BL];
    auto gload = [&](int kt) {
        const bool kok = kt * BK + ck * 8 < p.K;
#pragma unroll
        for (int i = 0; i < AL; ++i)
            ra[i] = (a_ok[i] && kok) ? *reinterpret_cast<const uint4 *>(a_src[i] + kt * BK) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < BL; ++i)
            rb[i] = (b_ok[i] && kok) ? *reinterpret_cast<const uint4 *>(b_src[i] + kt * BK) : make_uint4(0, 0, 0, 0);
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) *reinterpret_cast<uint4 *>(As + buf * BM * BK + a_dst[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < BL; ++i) *reinterpret_cast<uint4 *>(Bs + buf * BN * BK + b_dst[i]) = rb[i];
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (p.K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();

    // Fragment reads: lane l supplies row (l & 31) of a 32-row tile and the
    // 8 k values 8 (l >> 5) .. +7 of the current 16-wide k slice.
    const int frow = lane & 31;
    const int fsw = lane & 7;  // == row & 7 for every fragment row of this lane
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const f16 *as = As + cur * BM * BK + (wm * WM + frow) * BK;
        const f16 *bs = Bs + cur * BN * BK + (wn * WN + frow) * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = ((kk * 2 + (lane >> 5)) ^ fsw) << 3;
            f16x8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const f16x8 *>(as + i * 32 * BK + ch);
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const f16x8 *>(bs + j * 32 * BK + ch);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator register r of a 32x32 tile holds row
    // 8 (r >> 2) + 4 (lane >> 5) + (r & 3) and column lane & 31.
    const int hh = lane >> 5;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + (lane & 31);
        if (n >= p.N) continue;
        if constexpr (EPI == WENC_EPI_QKV) {
            const int slice = n / p.dmodel;
            const int c = n - slice * p.dmodel;
            const int h = c >> 6, e = c & 63;
            const float bn = p.bias[n];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int mb = m0 + wm * WM + i * 32 + 8 * g + 4 * hh;
                    if (slice < 2) {
                        f16 *dst = slice == 0 ? p.q : p.k;
                        const float sc = slice == 0 ? p.q_scale : 1.0f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = mb + r;
                            if (m < p.M) {
                                const uint32_t b = divu(m, p.t_div);
                                const uint32_t t = m - b * p.t_div.d;
                                dst[((int64_t(b) * p.H + h) * p.t_div.d + t) * 64 + e] =
                                    (f16)((acc[i][j][4 * g + r] + bn) * sc);
                            }
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = mb + r;
                            if (m < p.M) {
                                const uint32_t b = divu(m, p.t_div);
                                const uint32_t t = m - b * p.t_div.d;
                                p.vt[((int64_t(b) * p.H + h) * 64 + e) * p.ldvt + t] =
                                    (f16)(acc[i][j][4 * g + r] + bn);
                            }
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (m < p.M) epi_store<EPI>(p, m, n, acc[i][j][r]);
                }
        }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmP &base, int epi, hipStream_t s) {
    GemmP p = base;
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    const dim3 grid(p.tiles_m * p.tiles_n), block(256);
    switch (epi) {
        case WENC_EPI_GELU_F16: gemm_kernel<BM, BN, WM, WN, WENC_EPI_GELU_F16><<<grid, block, 0, s>>>(p); break;
        case WENC_EPI_CONV2: gemm_kernel<BM, BN, WM, WN, WENC_EPI_CONV2><<<grid, block, 0, s>>>(p); break;
        case WENC_EPI_RESID: gemm_kernel<BM, BN, WM, WN, WENC_EPI_RESID><<<grid, block, 0, s>>>(p); break;
        case WENC_EPI_QKV: gemm_kernel<BM, BN, WM, WN, WENC_EPI_QKV><<<grid, block, 0, s>>>(p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

const char *gemm_check(const wenc_gemm_args &a) {
    if (!a.A || !a.W || !a.bias) return "gemm: A, W and bias must be non-null";
    if (a.M < 0 || a.N <= 0 || a.K <= 0) return "gemm: need M >= 0, N > 0, K > 0";
    if (a.K % 8 || a.lda % 8 || a.ldw % 8 || a.a_batch_stride % 8)
        return "gemm: K, lda, ldw and a_batch_stride must be multiples of 8 (16-byte rows)";
    if (a.ldw < a.K) return "gemm: ldw < K";
    if (a.a_rows_per_batch <= 0 || a.a_rows_per_batch >= (1 << 16)) return "gemm: a_rows_per_batch out of [1, 65535]";
    if (a.M >= (1 << 24)) return "gemm: M must be < 2^24";
    switch (a.epilogue) {
        case WENC_EPI_GELU_F16:
            if (!a.C) return "gemm: C is null";
            if (a.c_rows_per_batch <= 0 || a.c_rows_per_batch >= (1 << 16)) return "gemm: c_rows_per_batch out of range";
            if (a.ldc < a.N) return "gemm: ldc < N";
            break;
        case WENC_EPI_CONV2:
            if (!a.C || !a.pos) return "gemm: C and pos must be non-null";
            if (a.pos_rows <= 0 || a.pos_rows >= (1 << 16)) return "gemm: pos_rows out of range";
            if (a.ldc < a.N) return "gemm: ldc < N";
            break;
        case WENC_EPI_RESID:
            if (!a.C) return "gemm: C is null";
            if (a.ldc < a.N) return "gemm: ldc < N";
            break;
        case WENC_EPI_QKV:
            if (!a.q || !a.k || !a.vt) return "gemm: q, k, vt must be non-null";
            if (a.n_head <= 0 || a.N != 3 * 64 * a.n_head) return "gemm: QKV needs N == 3 * 64 * n_head";
            if (a.T <= 0 || a.T >= (1 << 16) || a.M % a.T) return "gemm: QKV needs 0 < T < 65536 and M % T == 0";
            if (a.ldvt < a.T) return "gemm: ldvt < T";
            break;
        default:
            return "gemm: unknown epilogue";
    }
    return nullptr;
}

hipError_t launch_gemm(const wenc_gemm_args &a, hipStream_t s) {
    if (a.M == 0) return hipSuccess;
    GemmP p{};
    p.A = reinterpret_cast<const f16 *>(a.A);
    p.a_bs = a.a_batch_stride;
    p.a_div = make_divu(a.a_rows_per_batch);
    p.lda = a.lda;
    p.W = reinterpret_cast<const f16 *>(a.W);
    p.ldw = a.ldw;
    p.bias = a.bias;
    p.C = a.C;
    p.c_bs = a.c_batch_stride;
    p.c_div = make_divu(a.c_rows_per_batch > 0 ? a.c_rows_per_batch : 1);
    p.c_off = a.c_row_offset;
    p.ldc = a.ldc;
    p.pos = a.pos;
    p.pos_div = make_divu(a.pos_rows > 0 ? a.pos_rows : 1);
    p.q = reinterpret_cast<f16 *>(a.q);
    p.k = reinterpret_cast<f16 *>(a.k);
    p.vt = reinterpret_cast<f16 *>(a.vt);
    p.t_div = make_divu(a.T > 0 ? a.T : 1);
    p.H = a.n_head;
    p.ldvt = a.ldvt;
    p.dmodel = a.n_head * 64;
    p.q_scale = a.q_scale;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    return launch_cfg<128, 128, 64, 64>(p, a.epilogue, s);
}

}  // namespace wk
