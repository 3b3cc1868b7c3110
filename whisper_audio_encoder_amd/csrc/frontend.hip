// Whisper's log-mel frontend on gfx950: STFT power -> mel filters -> log10
// -> clamp at (window max - 8) -> (x + 4) / 4.
//
// CKE page ("How Audio Becomes Words"), section "The Frontend: Sound Becomes
// A Tensor": n_fft 400, hop 160, periodic Hann window, reflect padding, a
// 201 x 3000 power grid, n_mels area-normalised triangles on the Slaney mel
// scale, log10, a global -80 dB clamp (8 in log10 units, relative to the
// loudest value of the window) and the (x + 4) / 4 rescale.  Frames are
// centred (frame t starts at sample 160 t - 200 of the reflected signal) and
// the STFT's last frame is dropped, so a window of 160 F samples gives F
// frames; power is floored at 1e-10 before the logarithm.
//
// The STFT of a frame, X[k] = sum_j w[j] x[160 t - 200 + j] W^{jk} with
// W = e^{-2 pi i / 400}, is the 20 x 20 mixed-radix FFT the same section
// names.  With j = 20 a + c and k = p + 20 q (a, c, p in [0, 20)):
//   Y[p][c] = sum_a xw[20 a + c] W20^{a p}          (20-point DFTs of real data)
//   Z[p][c] = Y[p][c] W^{c p}                       (twiddles)
//   X[p + 20 q] = sum_c Z[p][c] W20^{c q}            (20-point DFTs over c)
// where W20 = W^20.  The data are real, so Y[20 - p] = conj(Y[p]) and only
// p <= 10 is formed; the second stage forms q = 0 .. 10 and keeps k <= 200.
// Both 20-point DFTs pair opposite inputs (j and 20 - j) so each output needs
// 9 products per part; cos and sin of 2 pi m / 20 are compile-time constants
// and products by 0 and +-1 are not issued.  fp32 throughout: the -80 dB clamp
// keeps bins down to 1e-8 of the peak power, below what fp16 resolves.
//
// The mel projection reads each triangle through a window of 16 n_ch bins
// that holds all of its non-zero weights (16 for the 80- and 128-filter
// banks, against 201 for a dense row), summed in increasing bin order.
//
// A 320-thread workgroup takes 16 frames of one window at a time: the
// samples, window, twiddles, the Z grid and the power rows live in LDS;
// thread (f, c) runs the first stage of frame f for column c, thread (f, p)
// the second stage for row p, and thread (g, m) sums filter m over every
// G-th frame from g, its weights in registers.
#include "common.h"
#include "kernels.h"

namespace wk {
namespace {

constexpr int NFFT = 400;
constexpr int HOP = 160;
constexpr int R = 20;                        // 400 = 20 x 20
constexpr int TF = 16;                       // frames per workgroup
constexpr int NT = TF * R;                   // 320 threads
constexpr int SPAN = HOP * (TF - 1) + NFFT;  // samples the 16 frames read: 2800
constexpr int ZS = R + 1;                    // float2 stride of a Z row: conflict-free row reads
constexpr int PS = 204;                      // power row stride (201 bins)
constexpr int XSZ = SPAN > TF * PS ? SPAN : TF * PS;  // samples, then (stage 2 on) power rows
constexpr int NLD = (SPAN + NT - 1) / NT;    // samples staged per thread
constexpr int NXW = (LOGMEL_MAX_EXTRA + NT - 1) / NT;  // extra mel weights staged per thread
constexpr int KF = 8;                        // frames per mel thread: at most 16 / G, G = 320 / n_mels >= 2
static_assert(2 * NT >= NFFT && NT >= 2 * LOGMEL_MAX_MELS, "one pass stages the tables; G >= 2");

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// cos and sin of 2 pi m / 20 (cos 18 deg, cos 36 deg, cos 54 deg, cos 72 deg).
constexpr float C1 = 0.951056516295153572f;
constexpr float C2 = 0.809016994374947424f;
constexpr float C3 = 0.587785252292473129f;
constexpr float C4 = 0.309016994374947424f;
__device__ constexpr float cos20(int m) {
    constexpr float t[R] = {1.f, C1, C2, C3, C4, 0.f, -C4, -C3, -C2, -C1, -1.f, -C1, -C2, -C3, -C4, 0.f, C4, C3, C2, C1};
    return t[m % R];
}
__device__ constexpr float sin20(int m) { return cos20(m + 15); }  // sin x = cos(x - pi / 2)

// acc + x k for a constant k known once the loops are unrolled: nothing for
// 0, an add or a subtract for +-1 (exact, as the fused form would be).
__device__ __forceinline__ float mac(float acc, float x, float k) {
    if (k == 0.0f) return acc;
    if (k == 1.0f) return acc + x;
    if (k == -1.0f) return acc - x;
    return __builtin_fmaf(x, k, acc);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Persistent: workgroup w takes jobs w, w + grid, ...; job j is frames
// 16 tile .. 16 tile + 15 of window b = j / tiles, tile = j % tiles.  The
// next job's samples are loaded into registers while the current one is
// computed.
__global__ void __launch_bounds__(NT)
logmel_kernel(const float *__restrict__ audio, int n_samples, int n_frames, int tiles, int jobs,
              const f32x2 *__restrict__ tab, const float *__restrict__ win, const float *__restrict__ mwt,
              const int *__restrict__ mstart, int nch, int n_mels, float *__restrict__ out,
              float *__restrict__ blkmax) {
    __shared__ float xs[XSZ];          // samples of the job; power rows from the second stage on
    __shared__ f32x2 zs[TF * R * ZS];  // Z[f][p][c]
    __shared__ f32x2 tw[NFFT];         // W^m = (cos, -sin) of 2 pi m / 400
    __shared__ float wn[NFFT];
    __shared__ float wx[LOGMEL_MAX_EXTRA];  // mel windows 1 .. nch - 1 of every filter
    __shared__ float wmax[NT / 64];
    const int tid = threadIdx.x;
    const int64_t limit_off = int64_t(HOP) * (n_frames - 1) + NFFT / 2;  // samples past this are read by no frame

    // Reflected sample loads of job j into registers (the edge sample itself
    // is not repeated; samples no valid frame reads are 0).
    float xv[NLD];
    auto load_job = [&](int j) {
        const int bj = j / tiles, t0 = (j - bj * tiles) * TF;
        const float *x = audio + int64_t(bj) * n_samples;
        const int64_t s0 = int64_t(HOP) * t0 - NFFT / 2;
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int p = tid + u * NT;
            const int64_t s = s0 + p;
            xv[u] = 0.0f;
            if (p < SPAN && s < limit_off) {
                const int64_t i = s < 0 ? -s : (s >= n_samples ? 2 * int64_t(n_samples - 1) - s : s);
                xv[u] = x[i];
            }
        }
    };

    // Mel work: thread (g, m), m = tid % n_mels, g = tid / n_mels < G, sums
    // filter m for frames g, g + G, ...  Its first 16 weights stay in
    // registers (the whole triangle for 72 or more filters).
    const int G = min(TF, NT / n_mels);
    const int g = tid / n_mels, m = tid - g * n_mels;
    const bool mel_lane = g < G;
    float w0[16];
    int ms = 0;
    if (mel_lane) {
        ms = mstart[m];
        const f32x4 *wp = reinterpret_cast<const f32x4 *>(mwt + int64_t(m) * nch * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = wp[q];
#pragma unroll
            for (int e = 0; e < 4; ++e) w0[4 * q + e] = v[e];
        }
    }
    // the tables (every global load here is issued before the first LDS store)
    f32x2 tv[2];
    float wv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + u * NT;
        if (i < NFFT) {
            tv[u] = tab[i];
            wv[u] = win[i];
        }
    }
    const int nx = n_mels * (nch - 1) * 16;  // <= LOGMEL_MAX_EXTRA
    float xw[NXW];
#pragma unroll
    for (int u = 0; u < NXW; ++u) {
        const int i = tid + u * NT;
        xw[u] = 0.0f;
        if (i < nx) xw[u] = mwt[(i >> 4) / (nch - 1) * nch * 16 + 16 + (i >> 4) % (nch - 1) * 16 + (i & 15)];
    }
    int job = blockIdx.x;
    if (job < jobs) load_job(job);
#pragma unroll
    for (int u = 0; u < NXW; ++u)
        if (tid + u * NT < nx) wx[tid + u * NT] = xw[u];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + u * NT;
        if (i < NFFT) {
            tw[i] = tv[u];
            wn[i] = wv[u];
        }
    }

    for (; job < jobs; job += gridDim.x) {
        const int b = job / tiles, tile = job - b * tiles, t0 = tile * TF;
#pragma unroll
        for (int u = 0; u < NLD; ++u)
            if (tid + u * NT < SPAN) xs[tid + u * NT] = xv[u];
        __syncthreads();
        if (job + int(gridDim.x) < jobs) load_job(job + gridDim.x);

        // First stage: thread (f, c), f = tid / 20.  Frame f's sample j sits
        // at xs[160 f + j].
        {
            const int f = tid / R, c = tid - f * R;
            const float *xf = xs + HOP * f + c;
            float xa[R];
#pragma unroll
            for (int a = 0; a < R; ++a) xa[a] = xf[R * a] * wn[R * a + c];
            float u[10], v[10];
#pragma unroll
            for (int a = 1; a < 10; ++a) {
                u[a] = xa[a] + xa[R - a];
                v[a] = xa[a] - xa[R - a];
            }
            float yr[11], yi[11];
#pragma unroll
            for (int p = 0; p <= 10; ++p) {
                float re = (p & 1) ? xa[0] - xa[10] : xa[0] + xa[10];
                float im = 0.0f;
#pragma unroll
                for (int a = 1; a < 10; ++a) {
                    re = mac(re, u[a], cos20(a * p));
                    im = mac(im, v[a], -sin20(a * p));
                }
                yr[p] = re;
                yi[p] = im;
            }
            f32x2 *zc = zs + f * R * ZS + c;
            zc[0] = f32x2{yr[0], yi[0]};
#pragma unroll
            for (int p = 1; p < R; ++p) {
                const float y_r = p <= 10 ? yr[p] : yr[R - p];
                const float y_i = p <= 10 ? yi[p] : -yi[R - p];
                const f32x2 w = tw[c * p];  // c p <= 361
                zc[p * ZS] = f32x2{y_r * w.x - y_i * w.y, __builtin_fmaf(y_r, w.y, y_i * w.x)};
            }
        }
        __syncthreads();

        // Second stage: thread (f, p) reads row p of frame f's Z (row index
        // f 20 + p = tid) and writes bins p + 20 q; q = 10 only exists for p = 0.
        {
            const int f = tid / R, p = tid - f * R;
            const f32x2 *zr = zs + tid * ZS;
            f32x2 z[R];
#pragma unroll
            for (int c = 0; c < R; ++c) z[c] = zr[c];
            f32x2 sm[10], df[10];
#pragma unroll
            for (int c = 1; c < 10; ++c) {
                sm[c] = z[c] + z[R - c];
                df[c] = z[c] - z[R - c];
            }
            float *pw = xs + f * PS;
#pragma unroll
            for (int q = 0; q <= 10; ++q) {
                float re = (q & 1) ? z[0].x - z[10].x : z[0].x + z[10].x;
                float im = (q & 1) ? z[0].y - z[10].y : z[0].y + z[10].y;
#pragma unroll
                for (int c = 1; c < 10; ++c) {
                    const float cs = cos20(c * q), sn = sin20(c * q);
                    re = mac(mac(re, sm[c].x, cs), df[c].y, sn);
                    im = mac(mac(im, sm[c].y, cs), df[c].x, -sn);
                }
                if (q < 10 || p == 0) pw[p + R * q] = __builtin_fmaf(re, re, im * im);
            }
        }
        __syncthreads();

        // Mel sums over bins ms .. ms + 16 nch - 1 in increasing order (the
        // weights are zero outside the triangle), then log10(max(m, 1e-10)).
        float mx = -3.0e38f;
        const int nvalid = min(TF, n_frames - t0);
        if (mel_lane) {
            float *o = out + (int64_t(b) * n_frames + t0) * n_mels + m;
#pragma unroll 2
            for (int k = 0; k < KF; ++k) {
                const int f = g + G * k;
                if (f >= nvalid) break;
                const float *pr = xs + f * PS + ms;
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < 16; ++j) acc = __builtin_fmaf(pr[j], w0[j], acc);
                for (int ch = 1; ch < nch; ++ch) {  // narrow filter banks only: later windows from LDS
                    const float *w = wx + (m * (nch - 1) + ch - 1) * 16;
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc = __builtin_fmaf(pr[16 * ch + j], w[j], acc);
                }
                const float v = __builtin_amdgcn_logf(fmaxf(acc, 1e-10f)) * 0.30102999566398120f;
                o[int64_t(f) * n_mels] = v;
                mx = fmaxf(mx, v);
            }
        }
        mx = wave_max(mx);
        if ((tid & 63) == 0) wmax[tid >> 6] = mx;
        __syncthreads();
        if (tid == 0) {
            float mm = wmax[0];
#pragma unroll
            for (int w = 1; w < NT / 64; ++w) mm = fmaxf(mm, wmax[w]);
            blkmax[int64_t(b) * tiles + tile] = mm;
        }
    }
}

// x = (max(x, M - 8) + 4) / 4 over window b, M the window's maximum.
__global__ void __launch_bounds__(256)
logmel_finish_kernel(float *__restrict__ out, const float *__restrict__ blkmax, int ntiles, int64_t n4) {
    __shared__ float part[4];
    const int b = blockIdx.y, tid = threadIdx.x;
    float mx = -3.0e38f;
    for (int i = tid; i < ntiles; i += 256) mx = fmaxf(mx, blkmax[int64_t(b) * ntiles + i]);
    mx = wave_max(mx);
    if ((tid & 63) == 0) part[tid >> 6] = mx;
    __syncthreads();
    const float lo = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3])) - 8.0f;
    f32x4 *o = reinterpret_cast<f32x4 *>(out) + int64_t(b) * n4;
    for (int64_t i = int64_t(blockIdx.x) * 256 + tid; i < n4; i += int64_t(gridDim.x) * 256) {
        f32x4 v = o[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (fmaxf(v[e], lo) + 4.0f) * 0.25f;
        o[i] = v;
    }
}

}  // namespace

int logmel_tiles(int n_frames) { return (n_frames + TF - 1) / TF; }

const char *logmel_check(int batch, int n_frames, int n_mels) {
    if (batch < 0 || batch > 65535) return "log_mel: batch outside [0, 65535]";
    if (n_frames < 2) return "log_mel: n_frames must be >= 2 (the reflect padding needs more than 200 samples)";
    if (int64_t(n_frames) * HOP >= (int64_t(1) << 31)) return "log_mel: window too long";
    if (n_mels <= 0 || n_mels > LOGMEL_MAX_MELS || n_mels % 8) return "log_mel: n_mels must be a multiple of 8, <= 128";
    return nullptr;
}

hipError_t launch_logmel(const float *audio, int batch, int n_frames, const float *tab, const float *win,
                         const float *mwt, const int *mstart, int nch, int n_mels, float *out, float *blkmax,
                         hipStream_t s) {
    if (batch == 0) return hipSuccess;
    if (nch < 1 || 16 * nch > 201 || n_mels * (nch - 1) * 16 > LOGMEL_MAX_EXTRA) return hipErrorInvalidValue;
    const int tiles = logmel_tiles(n_frames), jobs = tiles * batch;
    const int grid = int(std::min<long>(jobs, 2 * cu_count()));  // two workgroups fit a compute unit's LDS
    logmel_kernel<<<dim3(grid), dim3(NT), 0, s>>>(audio, n_frames * HOP, n_frames, tiles, jobs,
                                                  reinterpret_cast<const f32x2 *>(tab), win, mwt, mstart, nch,
                                                  n_mels, out, blkmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n4 = int64_t(n_frames) * n_mels / 4;
    int blocks = int((n4 + 1023) / 1024);
    if (blocks > 64) blocks = 64;
    logmel_finish_kernel<<<dim3(blocks, batch), dim3(256), 0, s>>>(out, blkmax, tiles, n4);
    return hipGetLastError();
}

}  // namespace wk
