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
// 32 of them and keeps them in registers.  Key tiles of 64 keys stream into
// LDS by direct buffer loads (double buffered), K as [key][64] and V^T as
// [dim][key slot], 16-byte chunks XOR-swizzled by row.  Each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_f16, so a lane holds 32 scores of ONE
// query: the row max and row sum are in-lane reductions plus one exchange
// with lane ^ 32.  The probabilities are then laid out as the B operand of
// O^T += V^T P^T, except that a lane holds its keys in runs of 4 (4 keys,
// skip 4).  The producer of V^T stores each 16-key group in exactly that
// order (key slot = key with bits 2 and 3 swapped), so one 16-byte LDS read
// gives a lane the 8 values of V^T it multiplies.
//
// q arrives multiplied by log2(e) / 8, so the softmax is evaluated with
// exp2 and no further scaling.  Keys at or beyond T get score -inf; their
// K rows read as zero (outside the buffer range) and their V^T slots must
// hold finite values (the producer writes zeros there).
#include "common.h"
#include "kernels.h"

namespace wk {

namespace {

constexpr int QT = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per tile
// s_waitcnt immediate with vmcnt = 0 and the other counters left alone
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int WAIT_VMCNT0 = 0x0f70;

// LDS chunk swizzle of a 128-byte row: conflict-free 16-byte reads for the 16
// lanes the LDS serves per cycle across its 64 banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t nbytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
    r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffff));
    r[2] = __builtin_amdgcn_readfirstlane(int(nbytes));
    r[3] = 0x00020000;
    return r;
}

// 1 KB global -> LDS transfer (lane i's 16 bytes land at lds + 16 i); an
// offset past the descriptor's range reads zero.  Inline assembly so the
// compiler does not serialise later LDS reads of the other buffer behind it;
// the loop orders it with s_waitcnt vmcnt(0) + barrier.  M0 carries the LDS
// address and is used by nothing else in this kernel.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, const f16 *lds, uint32_t voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) f16 *)lds)));
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(m0), "v"(voffset), "s"(rsrc)
        : "memory");
}

// At most 128 VGPRs, so four waves share each SIMD (the LDS allows five
// workgroups per CU); measured faster than three waves with no spill.
__global__ void __launch_bounds__(256, 4)
attn_kernel(const f16 *__restrict__ q, const f16 *__restrict__ k, const f16 *__restrict__ vt,
            f16 *__restrict__ ao, int T, int H, int ldvt) {
    // Workgroup ids are dealt round-robin over the 8 XCDs; renumber them so
    // each XCD gets a contiguous run, which keeps all query tiles of one
    // (batch, head) -- readers of the same K and V^T -- on one XCD's L2.
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int per = nwg >> 3, rem = nwg & 7, xcd = bid & 7, idx = bid >> 3;
    const int lid = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int nqt = (T + QT - 1) / QT;
    const int qt = lid % nqt, bhi = lid / nqt;
    const int h = bhi % H, b = bhi / H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, l32 = lane & 31;
    const int64_t bh = int64_t(b) * H + h;
    const f16 *Q = q + bh * T * 64;

    __shared__ __attribute__((aligned(1024))) f16 Ks0[KT * 64];
    __shared__ __attribute__((aligned(1024))) f16 Vs0[64 * KT];
    __shared__ __attribute__((aligned(1024))) f16 Ks1[KT * 64];
    __shared__ __attribute__((aligned(1024))) f16 Vs1[64 * KT];

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

    // Wait for the Q loads here, with a wait the compiler sees: its own
    // bookkeeping would otherwise place that wait inside the key loop, where
    // the hardware counter also holds the next key tile's transfers (issued
    // as inline assembly, invisible to the compiler), and every step would
    // stall until most of them had landed.
    __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);

    // Tile transfers: each wave moves rows 16 wave .. 16 wave + 15 of the K
    // tile and of the V^T tile (two 8-row groups each).  Lane i lands at row
    // 8 g + (i >> 3), chunk position i & 7, so it fetches logical chunk
    // (i & 7) ^ swz(row).
    const i32x4 rk = make_rsrc(k + bh * T * 64, uint32_t(T) * 128u);
    const i32x4 rv = make_rsrc(vt + bh * 64 * ldvt, uint32_t(ldvt) * 128u);
    uint32_t k_off[2], v_off[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int r = (wave * 2 + g) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        k_off[g] = uint32_t(r * 128 + c * 16);
        v_off[g] = uint32_t(r * ldvt * 2 + c * 16);
    }
    auto issue = [&](int kt, f16 *ks, f16 *vs) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            load_lds16(rk, ks + (wave * 2 + g) * 8 * 64, k_off[g] + uint32_t(kt) * (KT * 128));
            load_lds16(rv, vs + (wave * 2 + g) * 8 * 64, v_off[g] + uint32_t(kt) * (KT * 2));
        }
    };

    f32x16 o[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        o[0][r] = 0.f;
        o[1][r] = 0.f;
    }
    // Reference point of the softmax (base 2): probabilities are taken as
    // exp2(s - ref).  The fp16-representable part r16 of ref enters the
    // scores through one extra MFMA per 32-key tile, a constant A fragment
    // (1 in dimension 64 of every key, 0 in 65..79) against a B fragment
    // holding -r16 in dimension 64 of each query, so the subtraction costs
    // no VALU work; rlo = ref - r16 is non-zero only when |ref| > 2048 (then
    // the wave subtracts it explicitly).
    float ref = 0.f, rlo = 0.f, lsum = 0.f;
    f16x8 kone = {0, 0, 0, 0, 0, 0, 0, 0}, qref = {0, 0, 0, 0, 0, 0, 0, 0};
    if (hh == 0) kone[0] = (f16)1.0f;
    const int fsw = swz(l32);  // == swz(row) for every fragment row of this lane
    const int nkt = (T + KT - 1) / KT;

    auto step = [&](int kt, const f16 *ks, const f16 *vs) {
        // S^T tiles: rows = keys kt2*32 + 8 (r >> 2) + 4 hh + (r & 3), column = query l32.
        f32x16 s[2];
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt2][r] = 0.f;
            s[kt2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kone, qref, s[kt2], 0, 0, 0);  // -r16
            const f16 *kr = ks + (kt2 * 32 + l32) * 64;
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

        if (__any(rlo != 0.0f)) {
#pragma unroll
            for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kt2][r] -= rlo;
        }
        // s now holds score - ref.
        float mx = s[0][0];
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt2][r]);
        // Lazy rescaling: the reference point moves (to the tile maximum,
        // rounded to fp16) on the first tile and afterwards only when the
        // tile maximum exceeds it by more than 8 (log2 units), so the running
        // sum and O are rescaled rarely; probabilities taken against a stale
        // reference are at most 2^9, well inside fp16 and fp32.  The result
        // O / l is the same for any reference point.  Lanes l and l ^ 32 hold
        // halves of one query's keys and must share the reference, but their
        // maxima are exchanged only when some lane of the wave needs a move.
        if (kt == 0 || __any(mx > 8.0f)) {
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (kt == 0 || mx > 8.0f) {
                const float target = ref + mx;
                float nref, nlo;
                if (fabsf(target) <= 2048.0f) {  // fp16 rounding moves it by <= 1
                    nref = float((f16)target);
                    nlo = 0.0f;
                } else {
                    nref = target;
                    nlo = target;
                }
                const float shift = nref - ref;
                // lsum and o are still 0 on the first tile, where -shift may be
                // large enough for exp2 to overflow: scale by 0 there.
                const float alpha = kt == 0 ? 0.0f : __builtin_amdgcn_exp2f(-shift);
                lsum *= alpha;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    o[0][r] *= alpha;
                    o[1][r] *= alpha;
                }
#pragma unroll
                for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kt2][r] -= shift;
                ref = nref;
                rlo = nlo;
                if (hh == 0) qref[0] = (f16)(-(nref - nlo));
            }
        }
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt2][r] = __builtin_amdgcn_exp2f(s[kt2][r]);

        // O^T[dim][query] += V^T[dim][slots] P^T[slots][query], 16 keys per
        // MFMA: LDS chunk 2 s4 + hh of a V^T row holds exactly the 8 keys lane
        // half hh has probabilities for.  The row sum adds the same fp16
        // probabilities the MFMA consumes, two per instruction (dot with 1, 1,
        // accumulated in fp32).
        const f16x2 ones = {(f16)1.0f, (f16)1.0f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int kt2 = s4 >> 1, sg = s4 & 1;
            f16x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[i] = (f16)s[kt2][8 * sg + i];
#pragma unroll
            for (int i = 0; i < 4; ++i) lsum = __builtin_amdgcn_fdot2(f16x2{pb[2 * i], pb[2 * i + 1]}, ones, lsum, false);
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) {
                const int dim = ht * 32 + l32;
                const f16x8 va = *reinterpret_cast<const f16x8 *>(vs + dim * 64 + (((2 * s4 + hh) ^ fsw) << 3));
                o[ht] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb, o[ht], 0, 0, 0);
            }
        }
    };

    // Double-buffered key tiles; the loop is unrolled by two so each LDS
    // access names its buffer statically.
    issue(0, Ks0, Vs0);
#pragma unroll 1
    for (int kt = 0; kt < nkt; kt += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 1 < nkt) issue(kt + 1, Ks1, Vs1);
        step(kt, Ks0, Vs0);
        if (kt + 1 >= nkt) break;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 2 < nkt) issue(kt + 2, Ks0, Vs0);
        step(kt + 1, Ks1, Vs1);
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
    if (ldvt % KT || ldvt < T) return "attention: ldvt must be a multiple of 64 and >= T";
    if (int64_t((T + QT - 1) / QT) * n_head * batch >= (int64_t(1) << 31)) return "attention: grid too large";
    if (int64_t(ldvt) * 128 >= (int64_t(1) << 31) || int64_t(T) * 128 >= (int64_t(1) << 31))
        return "attention: T too large";
    return nullptr;
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *vt, uint16_t *ao,
                            int batch, int n_head, int T, int ldvt, hipStream_t s) {
    if (batch == 0) return hipSuccess;
    const dim3 grid(unsigned((T + QT - 1) / QT) * unsigned(n_head) * unsigned(batch)), block(256);
    attn_kernel<<<grid, block, 0, s>>>(reinterpret_cast<const f16 *>(q), reinterpret_cast<const f16 *>(k),
                                       reinterpret_cast<const f16 *>(vt), reinterpret_cast<f16 *>(ao), T, n_head,
                                       ldvt);
    return hipGetLastError();
}

}  // namespace wk
