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
// The STFT is a dense contraction per frame (X[t][k] = sum_n w[n] x[160 t -
// 200 + n] e^{-2 pi i k n / 400}), computed as fp32 MFMA (32x32x2) products:
// the frequency-by-sample basis (cos, -sin from a 400-entry table indexed by
// k n mod 400) is the A operand, the windowed samples the B operand.  The
// power tile that comes out is, register for register, already the B
// operand of the mel projection (summing k in the order the accumulator
// holds it), so power never leaves registers.  fp32 throughout: the -80 dB
// clamp keeps bins down to 1e-8 of the peak power, below what fp16 operands
// resolve.
#include "common.h"
#include "kernels.h"

namespace wk {
namespace {

constexpr int NFFT = 400;
constexpr int HOP = 160;
constexpr int NBIN = NFFT / 2 + 1;  // 201
constexpr int KT = 7;               // frequency tiles of 32
constexpr int KPAD = KT * 32;
static_assert(KPAD >= NBIN, "the frequency tiles cover every bin");
constexpr int TF = 32;              // frames per workgroup (one wave)
constexpr int SPAN = HOP * (TF - 1) + NFFT;  // samples the 32 frames read: 5360
constexpr int NSEG = (SPAN + HOP - 1) / HOP;  // 160-sample segments: 34
// Staged sample p sits at p + p / 160: each hop segment is followed by one
// pad float, so frame t starts at 161 t, whose LDS bank (161 t mod 64 =
// 33 t mod 64) differs for all 32 frames a B-operand read touches.
constexpr int XS = NSEG * (HOP + 1);

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// One workgroup = one wave = frames t0 .. t0+31 of window b.
__global__ void __launch_bounds__(64)
logmel_kernel(const float *__restrict__ audio, int n_samples, int n_frames, const f32x2 *__restrict__ tab,
              const float *__restrict__ win, const float *__restrict__ filt, int n_mels, int mtiles,
              float *__restrict__ out, float *__restrict__ blkmax) {
    __shared__ float xs[XS];
    __shared__ f32x2 tb[NFFT];
    __shared__ float wn[NFFT];
    const int b = blockIdx.y, tile = blockIdx.x, t0 = tile * TF, lane = threadIdx.x;
    const float *x = audio + int64_t(b) * n_samples;

    // Stage the samples, reflected about the first and last sample (the edge
    // sample itself is not repeated).  Samples no valid frame reads are 0.
    const int64_t s0 = int64_t(HOP) * t0 - NFFT / 2;
    const int64_t limit = int64_t(HOP) * (n_frames - 1) + NFFT / 2;
    for (int p = lane; p < SPAN; p += 64) {
        const int64_t s = s0 + p;
        float v = 0.0f;
        if (s < limit) {
            const int64_t i = s < 0 ? -s : (s >= n_samples ? 2 * int64_t(n_samples - 1) - s : s);
            v = x[i];
        }
        xs[p + p / HOP] = v;
    }
    for (int i = lane; i < NFFT; i += 64) {
        tb[i] = tab[i];
        wn[i] = win[i];
    }
    __syncthreads();

    // A operand (basis): lane l supplies frequency k = 32 kt + (l & 31) at
    // sample n = 2 s + (l >> 5).  B operand (samples): lane l supplies frame
    // t = l & 31 at the same n.  Accumulator register r of lane l then holds
    // frame l & 31 and frequency 32 kt + 8 (r >> 2) + 4 (l >> 5) + (r & 3).
    const int t = lane & 31, hh = lane >> 5;
    const float *xb = xs + (HOP + 1) * t + hh;
    const float *wb = wn + hh;
    f32x16 mel[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mel[i][r] = 0.0f;

#pragma unroll 1
    for (int kt = 0; kt < KT; ++kt) {
        const uint32_t k = uint32_t(kt * 32 + t);
        const uint32_t dk = (2 * k) % NFFT;
        uint32_t idx = (k * uint32_t(hh)) % NFFT;
        f32x16 re, im;
#pragma unroll
        for (int r = 0; r < 16; ++r) re[r] = im[r] = 0.0f;
        auto step = [&](int s, int seg) {
            const float bx = xb[2 * s + seg] * wb[2 * s];
            const f32x2 a = tb[idx];
            re = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bx, re, 0, 0, 0);
            im = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bx, im, 0, 0, 0);
            idx += dk;
            idx = min(idx, idx - uint32_t(NFFT));  // idx - 400 wraps above 2^31 while idx < 400
        };
        // n = 2 s + (l >> 5) crosses a hop segment (one pad float) at s = 80 and 160
#pragma unroll 8
        for (int s = 0; s < 80; ++s) step(s, 0);
#pragma unroll 8
        for (int s = 80; s < 160; ++s) step(s, 1);
#pragma unroll 8
        for (int s = 160; s < 200; ++s) step(s, 2);

        f32x16 pw;
#pragma unroll
        for (int r = 0; r < 16; ++r) pw[r] = re[r] * re[r] + im[r] * im[r];
        // Mel projection: A' = filters (lane l: filter 32 mt + (l & 31)), B' =
        // power; MFMA step r sums frequency 32 kt + 8 (r >> 2) + 4 h + (r & 3)
        // for lane half h, exactly the frequency pw[r] holds.
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt >= mtiles) break;
            const float *fr = filt + (mt * 32 + t) * KPAD + kt * 32 + 4 * hh;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 f = *reinterpret_cast<const f32x4 *>(fr + 8 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    mel[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(f[e], pw[4 * g + e], mel[mt], 0, 0, 0);
            }
        }
    }

    // log10(max(m, 1e-10)) in the mel accumulators' layout: lane l holds
    // frame t0 + (l & 31) and filters 32 mt + 8 g + 4 h + e, stored as runs of 4.
    const int frame = t0 + t;
    float mx = -3.0e38f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        if (mt >= mtiles) break;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int m = mt * 32 + 8 * g + 4 * hh;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = __builtin_amdgcn_logf(fmaxf(mel[mt][4 * g + e], 1e-10f)) * 0.30102999566398120f;
            if (frame < n_frames && m < n_mels) {
                *reinterpret_cast<f32x4 *>(out + (int64_t(b) * n_frames + frame) * n_mels + m) = v;
                mx = fmaxf(mx, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
            }
        }
    }
    mx = wave_max(mx);
    if (lane == 0) blkmax[int64_t(b) * gridDim.x + tile] = mx;
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
    if (n_mels <= 0 || n_mels > 128 || n_mels % 8) return "log_mel: n_mels must be a multiple of 8, <= 128";
    return nullptr;
}

hipError_t launch_logmel(const float *audio, int batch, int n_frames, const float *tab, const float *win,
                         const float *filt, int n_mels, float *out, float *blkmax, hipStream_t s) {
    if (batch == 0) return hipSuccess;
    const int tiles = logmel_tiles(n_frames);
    logmel_kernel<<<dim3(tiles, batch), dim3(64), 0, s>>>(audio, n_frames * HOP, n_frames,
                                                          reinterpret_cast<const f32x2 *>(tab), win, filt, n_mels,
                                                          (n_mels + 31) / 32, out, blkmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n4 = int64_t(n_frames) * n_mels / 4;
    int blocks = int((n4 + 1023) / 1024);
    if (blocks > 64) blocks = 64;
    logmel_finish_kernel<<<dim3(blocks, batch), dim3(256), 0, s>>>(out, blkmax, tiles, n4);
    return hipGetLastError();
}

}  // namespace wk
