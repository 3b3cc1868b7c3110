// Greedy token choice on the device, for gfx950.
//
// Greedy decoding takes, per sequence and step, the index of the largest of
// the vocabulary's logits (51865 for Whisper); the whisper README
// ("Performance and memory") names fetching all of them to the host for
// that search as one of the two costs it removed from a decode step, by
// reducing on the device and returning one integer.  Per row r:
//   out[r] = min { i : logits[r][i] = max_j logits[r][j] }
// where a NaN counts as larger than every number (the first NaN wins) and
// -0.0 equals +0.0.
//
// Each candidate becomes one 64-bit key: the high word is the value mapped
// to an unsigned integer that orders like the float (NaN mapped above +inf,
// -0.0 folded onto +0.0), the low word is ~index, so that the largest key
// is the smallest index among the maxima.  Max over keys is associative and
// commutative, so the result does not depend on how the row is split.
//
// Pass 1 (amax_partial): a workgroup of 256 lanes takes 2048 consecutive
// logits of a row (8 coalesced 4-byte loads per lane, all issued before the
// first compare) and writes its largest key.  Pass 2 (amax_merge): one wave
// per row takes the maximum over the row's chunk keys and writes the index.
// A row of at most 2048 logits is finished in pass 1.  The work is bound by
// reading the logits once (HBM), and at one decode step's size by launch
// latency.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace wk {

namespace {

// Chunk keys of the allocation-free entry point (wenc_argmax_noalloc): one
// array per device, part of the code object, so the call needs no device
// allocation.  Host code must not pass the array's name to a kernel (on the
// host it is only a stand-in for the symbol): static_scratch() looks up its
// device address once per device and every launch uses that.
static __device__ __align__(256) uint64_t scratch[ARGMAX_STATIC_KEYS];

constexpr int AM_THREADS = 256;
constexpr int AM_PER_LANE = 8;
constexpr int AM_CHUNK = AM_THREADS * AM_PER_LANE;  // logits per workgroup of pass 1

__device__ __forceinline__ uint64_t am_key(float x, uint32_t i) {
    uint32_t b = __float_as_uint(x);
    uint32_t k;
    if (x != x) {
        k = 0xffffffffu;  // NaN: above +inf (0xff800000 after the mapping)
    } else {
        if (b == 0x80000000u) b = 0u;  // -0.0 -> +0.0
        k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
    return (uint64_t(k) << 32) | uint64_t(~i);
}

__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t lo = __shfl_xor(uint32_t(v), o), hi = __shfl_xor(uint32_t(v >> 32), o);
        v = max64(v, (uint64_t(hi) << 32) | lo);
    }
    return v;
}

// grid: rows x nc workgroups (chunk fastest).  With nc == 1 the index is
// written directly to out; otherwise the key goes to part[row * nc + chunk].
__global__ void __launch_bounds__(AM_THREADS)
amax_partial(const float *__restrict__ logits, int64_t ld, int n, int nc, uint64_t *__restrict__ part,
             int32_t *__restrict__ out) {
    const int c = blockIdx.x % nc;
    const int64_t row = blockIdx.x / nc;
    const float *x = logits + row * ld;
    const int base = c * AM_CHUNK + threadIdx.x;
    float v[AM_PER_LANE];
#pragma unroll
    for (int j = 0; j < AM_PER_LANE; ++j) {
        const int i = base + j * AM_THREADS;
        v[j] = i < n ? x[i] : 0.f;
    }
    uint64_t key = 0;  // below every candidate (the smallest is -inf's, 0x007fffff in the high word)
#pragma unroll
    for (int j = 0; j < AM_PER_LANE; ++j) {
        const int i = base + j * AM_THREADS;
        if (i < n) key = max64(key, am_key(v[j], uint32_t(i)));
    }
    key = wave_max64(key);
    __shared__ uint64_t wkey[AM_THREADS / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) wkey[wave] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t k = wkey[0];
#pragma unroll
        for (int w = 1; w < AM_THREADS / 64; ++w) k = max64(k, wkey[w]);
        if (nc == 1)
            out[row] = int32_t(~uint32_t(k));
        else
            part[row * nc + c] = k;
    }
}

__global__ void __launch_bounds__(64)
amax_merge(const uint64_t *__restrict__ part, int nc, int32_t *__restrict__ out) {
    const int64_t row = blockIdx.x;
    uint64_t k = 0;
    for (int c = threadIdx.x; c < nc; c += 64) k = max64(k, part[row * nc + c]);
    k = wave_max64(k);
    if (threadIdx.x == 0) out[row] = int32_t(~uint32_t(k));
}

}  // namespace

int argmax_chunks(int n_vocab) { return int((int64_t(n_vocab) + AM_CHUNK - 1) / AM_CHUNK); }

hipError_t static_scratch(uint64_t **keys) {
    static std::mutex mu;
    static uint64_t *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // with `dev` current: each device holds its own copy of the array
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<uint64_t *>(p);
    }
    *keys = addr[dev];
    return hipSuccess;
}

const char *argmax_check(int rows, int n_vocab, int64_t ld) {
    if (rows < 0) return "argmax: rows must be >= 0";
    if (n_vocab < 1 || n_vocab > (1 << 30)) return "argmax: n_vocab must be in [1, 2^30]";
    if (ld < n_vocab) return "argmax: ld must be >= n_vocab";
    if (int64_t(rows) * argmax_chunks(n_vocab) >= (int64_t(1) << 31)) return "argmax: grid too large";
    return nullptr;
}

hipError_t launch_argmax(const float *logits, int rows, int n_vocab, int64_t ld, uint64_t *part, int32_t *out,
                         hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int nc = argmax_chunks(n_vocab);
    amax_partial<<<dim3(unsigned(int64_t(rows) * nc)), dim3(AM_THREADS), 0, s>>>(logits, ld, n_vocab, nc, part, out);
    if (nc > 1) amax_merge<<<dim3(unsigned(rows)), dim3(64), 0, s>>>(part, nc, out);
    return hipGetLastError();
}

}  // namespace wk
