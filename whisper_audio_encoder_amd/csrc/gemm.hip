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
// is exactly the operand layout v_mfma_f32_16x16x32_f16 reads per lane.
//
// Structure (details at each step below).  A workgroup of NW wave64s owns a
// BM x BN output tile and walks K in steps of 64 (two MFMA k slices of 32).
// Each step is moved from global memory straight into LDS by
// buffer_load ... lds (no VGPR staging); a buffer offset with bit 31 set
// lies beyond the descriptor's range and reads as zero, which pads the M, N
// and K tails without branches.  Within LDS, 16-byte chunks are XOR-swizzled
// by row so that fragment reads are free of bank conflicts; the direct loads
// produce that layout by choosing which global chunk each lane fetches.  The
// A part of a step has three LDS buffers and the W part two.  The 128 x 128
// kernel issues A transfers three steps ahead of their use and W transfers
// two, with one barrier per step.  The 256 x 256 kernel runs a ping-pong
// schedule: the two waves sharing a SIMD work a phase apart, one issuing a
// step's MFMAs while the other reads its fragments from LDS and issues
// transfers (details at the main loop).  The MFMA takes W as its A operand and A^T as its B operand, so
// each lane ends up owning one output row and runs of 4 consecutive output
// columns, which the epilogues store as 8- or 16-byte vectors.
//
// Workgroup ids are remapped so that each XCD (ids are dealt round-robin
// over the 8 XCDs) receives a contiguous run of tiles, ordered in groups of
// a few tile rows (tile_coords), so tiles sharing A rows or W rows share
// that XCD's L2.
#include <algorithm>
#include <atomic>
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace wk {

namespace {

constexpr int BK = 64;
constexpr uint32_t OOB = 0x80000000u;  // buffer offset beyond num_records: reads 0

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
    int c_run8;  // GELU fp16: rows of C at non-decreasing addresses, N % 8 == 0 and a tile's rows
                 // within 2 GiB of its first: the epilogue stores through one buffer descriptor
    int qk_run8; // QKV: a tile's q and k rows within 2 GiB of its first row's: the same
    const float *pos;
    DivU pos_div;
    f16 *q, *k, *vt;
    f16 *C2;
    int n_split;
    int a_valid;  // rows r of a batch item with r % a_rows_per_batch >= a_valid read as zero
    int T;        // QKV: keys per batch item (the row space is padded to t_div.d = T rounded up to 16)
    DivU t_div;
    int H, ldvt, dmodel;
    float q_scale;
    int M, N, K;
    int m_begin;  // first row this launch covers (rows m_begin .. M-1)
    int tiles_m, tiles_n;
};

// Group height GM: a run of consecutive tiles covers GM tile rows across all
// tile columns, and an XCD runs about 32 consecutive tiles at once, so GM x
// tiles_n near 32 lets one round read each A row panel into that XCD's L2
// for all its column tiles.  Measured on the encoder's projections (d 1280):
// 6 for five columns (fc2, out_proj, conv2: fc2 -3.5%), 4 for 15 to 20
// (q|k|v, fc1: -1 to -2%), 8 otherwise (unchanged at d 768).
__device__ __forceinline__ void tile_coords(int bid, int nwg, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int per = nwg >> 3, rem = nwg & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    const int lid = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int GM = tiles_n <= 5 ? 6 : (tiles_n >= 15 ? 4 : 8);
    const int group_size = GM * tiles_n;
    const int g = lid / group_size;
    const int first_m = g * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in = lid - g * group_size;
    tm = first_m + in % gm;
    tn = in / gm;
}

// Element offset of A row m (batch remap for the conv stem's frame windows).
__device__ __forceinline__ int64_t a_row(const GemmP &p, uint32_t m) {
    const uint32_t bi = divu(m, p.a_div);
    return int64_t(bi) * p.a_bs + int64_t(m - bi * p.a_div.d) * p.lda;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + 2 GiB): raw (stride 0), so an offset
// at or past num_records reads as zero.
__device__ __forceinline__ i32x4 make_rsrc(const void *base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
    r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffff));
    r[2] = 0x7fffffff;
    r[3] = 0x00020000;
    return r;
}

// One 16-byte-per-lane global -> LDS transfer of 1 KB: lane i's data lands
// at LDS byte address lds + 16 i.  Written as inline assembly so that the
// compiler does not see an LDS store: it would otherwise wait for every such
// transfer before later LDS reads of the other buffer.  The main loop orders
// the transfers itself (s_waitcnt vmcnt(0) + barrier before any wave reads
// the buffer they fill).  M0 carries the LDS address; nothing else in these
// kernels uses M0.  The descriptor words go through readfirstlane so that
// the operand stays in scalar registers inside branches on the wave index.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t lds, uint32_t voffset) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset),
          "s"(i32x4{__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])})
        : "memory");
}

// LDS byte address of a __shared__ object (the generic-to-LDS cast carries a
// null check, so it is taken once per kernel).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)p)));
}

// LDS chunk swizzle.  A tile row is 128 B (8 chunks of 16 B); logical chunk c
// of row r is stored at chunk position c ^ swz(r).  The LDS serves a 16-byte
// read for 16 lanes per cycle across 64 banks, i.e. two 128-byte rows'
// worth: the 16 rows read together must cover the 16 (row parity, chunk
// position) pairs, which this XOR on bits 1..3 of the row guarantees.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

__device__ __forceinline__ uint32_t vt_slot(uint32_t t) { return (t & ~12u) | ((t & 4u) << 1) | ((t & 8u) >> 1); }

// Row-major epilogue stores of the LDS-staged path: 8 consecutive fp16
// outputs (n .. n+7 of row m, n + 4 <= N) or 4 consecutive fp32 outputs.
__device__ __forceinline__ void store_f16_run(f16 *dst, int n, int N, f16x8 o) {
    if (n + 8 <= N) {
        *reinterpret_cast<f16x8 *>(dst) = o;
    } else {
        *reinterpret_cast<f16x4 *>(dst) = f16x4{o[0], o[1], o[2], o[3]};
    }
}

template <int EPI>
__device__ __forceinline__ void epi_row8(const GemmP &p, int m, int n, f16x8 o) {
    if constexpr (EPI == WENC_EPI_GELU_F16) {
        const uint32_t bi = divu(m, p.c_div);
        const uint32_t r = m - bi * p.c_div.d;
        store_f16_run(static_cast<f16 *>(p.C) + int64_t(bi) * p.c_bs + int64_t(r + p.c_off) * p.ldc + n, n, p.N, o);
    } else if constexpr (EPI == WENC_EPI_KV) {
        if (n + 8 <= p.n_split || n >= p.n_split) {
            const bool hi = n >= p.n_split;
            f16 *C = (hi ? p.C2 : static_cast<f16 *>(p.C)) + int64_t(m) * p.ldc + (hi ? n - p.n_split : n);
            store_f16_run(C, n, p.N, o);
        } else {  // a run straddling n_split (n_split % 8 == 4)
            *reinterpret_cast<f16x4 *>(static_cast<f16 *>(p.C) + int64_t(m) * p.ldc + n) = f16x4{o[0], o[1], o[2], o[3]};
            if (n + 4 < p.N)
                *reinterpret_cast<f16x4 *>(p.C2 + int64_t(m) * p.ldc) = f16x4{o[4], o[5], o[6], o[7]};
        }
    } else if constexpr (EPI == WENC_EPI_QKV) {  // q or k columns; pad rows (t >= T) are not stored
        const int slice = n / p.dmodel;
        const int c = n - slice * p.dmodel;
        const uint32_t bb = divu(m, p.t_div);
        const uint32_t t = m - bb * p.t_div.d;
        if (t >= uint32_t(p.T)) return;
        f16 *dst = slice == 0 ? p.q : p.k;
        *reinterpret_cast<f16x8 *>(dst + ((int64_t(bb) * p.H + (c >> 6)) * p.T + t) * 64 + (c & 63)) = o;
    }
}

// TAG only separates otherwise identical instantiations (fc1 from conv1,
// fc2 from out_proj) so that a kernel trace names each projection.
// A 256 x 256 tile runs one workgroup per CU (its LDS allows one); the
// 128 x 128 kernel is held to two workgroups per CU (its LDS allows two).
// (A 4-wave 256 x 256 kernel with 128 x 128 per wave, accumulators in
// AGPRs, compiles from this template too; it measured 10-20% slower.)
template <int BM, int BN, int WM, int WN, int NW, int EPI, int TAG, int PP>
__global__ void __launch_bounds__(NW * 64, (NW >= 8 || BM >= 256) ? 1 : 2)
gemm_kernel(const GemmP p) {
    constexpr int WAVES_N = BN / WN;
    static_assert((BM / WM) * (BN / WN) == NW, "wave grid");
    constexpr int TM = WM / 16, TN = WN / 16;
    // Waves that issue the direct loads.  With 8 waves two share each SIMD
    // (wave w runs on SIMD w % 4); only waves 0..3 load, so their partners
    // issue MFMAs without queueing behind vector-memory instructions
    // (4-7 % faster on 24000x5120x1280 and 8192^3 than all 8 loading).
    constexpr int LW = NW >= 8 ? NW / 2 : NW;
    constexpr int AG = BM / 8 / LW;  // 8-row groups of A each loading wave moves per step
    constexpr int BG = BN / 8 / LW;
    static_assert(AG >= 1 && BG >= 1, "each loading wave moves at least one group");
    constexpr int STAGE = (BM + BN) * BK;  // halves per LDS stage
    constexpr int ASZ = BM * BK;           // halves of the A part of a stage
    __shared__ __attribute__((aligned(1024))) f16 smem0[STAGE];  // A buffer 0 | W buffer 0
    __shared__ __attribute__((aligned(1024))) f16 smem1[STAGE];  // A buffer 1 | W buffer 1
    __shared__ __attribute__((aligned(1024))) f16 smemA2[ASZ];   // A buffer 2

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS addresses stay scalar
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = p.m_begin + tm * BM, n0 = tn * BN;

    // Direct loads: one instruction moves 8 tile rows x 128 B; lane i lands at
    // row r = 8 g + (i >> 3), chunk position i & 7, so it fetches logical
    // chunk (i & 7) ^ sw(r).
    // Tile base: the row of m0, or for a pad row (QKV) the start of the next
    // batch item, so that every row offset below is non-negative.
    const uint32_t b0 = divu(m0, p.a_div);
    const int64_t a0 = int64_t(b0) * p.a_bs + int64_t(min(int(m0 - b0 * p.a_div.d), p.a_valid)) * p.lda;
    const int lw = wave < LW ? wave : 0;  // offsets of the waves that load
    uint32_t a_off[AG], a_ch[AG];
#pragma unroll
    for (int g = 0; g < AG; ++g) {
        const int r = (lw * AG + g) * 8 + (lane >> 3);
        a_ch[g] = (lane & 7) ^ swz(r);
        const int m = m0 + r;
        const bool ok = m < p.M && int(m - divu(m, p.a_div) * p.a_div.d) < p.a_valid;
        a_off[g] = ok ? uint32_t((a_row(p, m) - a0) * 2) + a_ch[g] * 16 : OOB;
    }
    uint32_t b_off[BG], b_ch[BG];
#pragma unroll
    for (int g = 0; g < BG; ++g) {
        const int r = (lw * BG + g) * 8 + (lane >> 3);
        b_ch[g] = (lane & 7) ^ swz(r);
        b_off[g] = n0 + r < p.N ? uint32_t(r * p.ldw * 2 + b_ch[g] * 16) : OOB;
    }
    const i32x4 ra = make_rsrc(p.A + a0);
    const i32x4 rb = make_rsrc(p.W + int64_t(n0) * p.ldw);

    const uint32_t lds0 = lds_addr(smem0), lds1 = lds_addr(smem1), lds2 = lds_addr(smemA2);
    const uint32_t la0 = lds0, la1 = lds1, la2 = lds2;                 // A buffers
    const uint32_t lw0 = lds0 + ASZ * 2, lw1 = lds1 + ASZ * 2;         // W buffers
    // Direct loads of K step kt: the A part into the A buffer at LDS byte
    // address st, the W part into the W buffer at st.  Steps that lie wholly
    // inside K (every step when K % 64 == 0) skip the K-tail test.
    auto issueA = [&](int kt, uint32_t st) __attribute__((always_inline)) {
        if (wave >= LW) return;
        const uint32_t kb = uint32_t(kt) * (BK * 2);
        if ((kt + 1) * BK <= p.K) {
#pragma unroll
            for (int g = 0; g < AG; ++g) load_lds16(ra, st + (lw * AG + g) * 8 * BK * 2, a_off[g] + kb);
        } else {
#pragma unroll
            for (int g = 0; g < AG; ++g) {
                const uint32_t kflag = (kt * BK + int(a_ch[g]) * 8 < p.K) ? 0u : OOB;
                load_lds16(ra, st + (lw * AG + g) * 8 * BK * 2, (a_off[g] | kflag) + kb);
            }
        }
    };
    auto issueW = [&](int kt, uint32_t st) __attribute__((always_inline)) {
        if (wave >= LW) return;
        const uint32_t kb = uint32_t(kt) * (BK * 2);
        if ((kt + 1) * BK <= p.K) {
#pragma unroll
            for (int g = 0; g < BG; ++g) load_lds16(rb, st + (lw * BG + g) * 8 * BK * 2, b_off[g] + kb);
        } else {
#pragma unroll
            for (int g = 0; g < BG; ++g) {
                const uint32_t kflag = (kt * BK + int(b_ch[g]) * 8 < p.K) ? 0u : OOB;
                load_lds16(rb, st + (lw * BG + g) * 8 * BK * 2, (b_off[g] | kflag) + kb);
            }
        }
    };

    // Accumulator (i, j) is the 16 x 16 block of rows 16 i and columns 16 j of
    // the wave's tile; its register r holds row (lane & 15) and column
    // 4 (lane >> 4) + r.  Every accumulator starts at its column's bias, so
    // the epilogues add none.  The bias loads are issued first, as inline
    // assembly like the direct loads, and the prologue's own wait covers
    // them (transfers complete in issue order).  Issued as ordinary loads,
    // they would make the compiler wait for them just before the first
    // step, where the hardware counter also holds the direct loads of the
    // next two steps (invisible to it), so the first step would not start
    // until those had landed.
    const int hh = lane >> 4;
    f32x4 bias[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + 4 * hh;
        const float *bp = p.bias + min(n, p.N - 4);  // a column past N loads column N - 4 and is zeroed below
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(bias[j]) : "v"(bp) : "memory");
    }
    f32x4 acc[TM][TN];

    // Fragment reads (v_mfma_f32_16x16x32_f16 operands): lane supplies row
    // (lane & 15) of a 16-row block and k values 8 (lane >> 4) .. +7 of the
    // current 32-wide slice, one 16-byte LDS read per block.
    const int frow = lane & 15;
    const int fsw = swz(lane & 15);  // == swz(row) for every fragment row of this lane
    static_assert(BK == 64, "the main loop walks two 32-wide k slices per step");

    // Main loop.  A step of 64 k is two slices of 32.  Fragments roll: the
    // A-side fragment of block row i for the next slice is read as soon as
    // the MFMAs of block row i of this slice are issued, into the same
    // registers, and the W-side fragments alternate between two sets; so
    // every read has most of a slice of MFMAs to land before its consumer,
    // with one A-side set live.  The barrier that publishes step kt+1 sits
    // between the two slices of step kt: slice 1's fragments are already in
    // registers, so its MFMAs overlap the barrier and the reads of step
    // kt+1's slice 0, and the direct loads of W for step kt+2 and of A for
    // step kt+3 go into the buffers step kt has just released.  (The last
    // step's slice 1 reads idle buffers; those fragments are not used.)
    const int nk = (p.K + BK - 1) / BK;
    if constexpr (PP) {
        static_assert(BM == 256 && BN == 256 && WM == 128 && WN == 64 && NW == 8, "ping-pong: 256 x 256, 8 waves");
        // Ping-pong schedule.  Wave w runs on SIMD w % 4, so waves w and
        // w + 4 share a SIMD: group 0 (waves 0..3, tile rows 0..127) and
        // group 1 (waves 4..7, rows 128..255) have one wave on each SIMD.
        // Every wave runs the same loop, per k step j: a memory phase (its
        // share of a later step's direct loads, then the fragments of step
        // j from LDS), a barrier, a compute phase (the step's 64 MFMAs), a
        // barrier.  Group 1 passes one extra barrier before the loop, so
        // its phases run one slot behind group 0's: while one wave of a
        // SIMD issues MFMAs, the other's LDS reads are in flight.  Step j
        // is read by group 0 in slot 2j and by group 1 in slot 2j + 1.
        // Group 0 moves W: in its memory phase of step j, W of step j + 1
        // into the W buffer step j - 1 has freed; it waits for it after its
        // compute phase of step j.  Group 1 moves A: in its memory phase of
        // step j, A of step j + 2 into the A buffer step j - 1 has freed;
        // it waits for A of step j + 1 at the end of that phase.  Either
        // way a step's data has landed before the barrier that opens slot
        // 2j, where group 0 first reads it.  The compute phase reads the A
        // side of the second k slice itself (see pcomp).
        const int grp = wm;
        const int lw4 = wave & 3;
        uint32_t poff[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int r = (lw4 * 8 + g) * 8 + (lane >> 3);
            const uint32_t ch = uint32_t((lane & 7) ^ swz(r));
            uint32_t off;
            if (grp == 0) {
                off = n0 + r < p.N ? uint32_t(r * p.ldw * 2) + ch * 16 : OOB;
            } else {
                const int m = m0 + r;
                const bool ok = m < p.M && int(m - divu(m, p.a_div) * p.a_div.d) < p.a_valid;
                off = ok ? uint32_t((a_row(p, m) - a0) * 2) + ch * 16 : OOB;
            }
            poff[g] = off;
        }
        const i32x4 prs = grp == 0 ? rb : ra;
        // this wave's share of its group's operand for step kt, into the
        // LDS buffer at byte address st
        auto pissue = [&](int kt, uint32_t st) __attribute__((always_inline)) {
            const uint32_t kb = uint32_t(kt) * (BK * 2);
            if ((kt + 1) * BK <= p.K) {
#pragma unroll
                for (int g = 0; g < 8; ++g) load_lds16(prs, st + (lw4 * 8 + g) * 8 * BK * 2, poff[g] + kb);
            } else {
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    const int r = (lw4 * 8 + g) * 8 + (lane >> 3);
                    const int ch = (lane & 7) ^ swz(r);
                    const uint32_t kflag = (kt * BK + ch * 8 < p.K) ? 0u : OOB;
                    load_lds16(prs, st + (lw4 * 8 + g) * 8 * BK * 2, (poff[g] | kflag) + kb);
                }
            }
        };
        // Fragments: the memory phase reads the A side of slice 0 and the W
        // side of both slices; the compute phase reads the A side of slice 1
        // into the registers of slice 0's, block row by block row, as soon
        // as that row's slice-0 MFMAs are issued (a wave holds one A-side
        // set: the registers of a whole step's fragments would not fit).
        f16x8 pa[TM], pb0[TN], pb1[TN];
        const int pch0 = ((lane >> 4) ^ fsw) << 3, pch1 = ((4 + (lane >> 4)) ^ fsw) << 3;
        auto pmem = [&](const f16 *asrc, const f16 *wsrc) __attribute__((always_inline)) {
            const f16 *as = asrc + (wm * WM + frow) * BK;
            const f16 *bs = wsrc + (wn * WN + frow) * BK;
#pragma unroll
            for (int i = 0; i < TM; ++i) pa[i] = *reinterpret_cast<const f16x8 *>(as + i * 16 * BK + pch0);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                pb0[j] = *reinterpret_cast<const f16x8 *>(bs + j * 16 * BK + pch0);
                pb1[j] = *reinterpret_cast<const f16x8 *>(bs + j * 16 * BK + pch1);
            }
        };
        auto pcomp = [&](const f16 *asrc) __attribute__((always_inline)) {
            const f16 *as = asrc + (wm * WM + frow) * BK;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb0[j], pa[i], acc[i][j], 0, 0, 0);
                pa[i] = *reinterpret_cast<const f16x8 *>(as + i * 16 * BK + pch1);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb1[j], pa[i], acc[i][j], 0, 0, 0);
        };
        const f16 *A0 = smem0, *A1 = smem1, *A2 = smemA2, *W0 = smem0 + ASZ, *W1 = smem1 + ASZ;
        const uint32_t la0 = lds_addr(smem0), la1 = lds_addr(smem1), la2 = lds_addr(smemA2);
        const uint32_t lw0 = la0 + ASZ * 2, lw1 = la1 + ASZ * 2;
        // prologue: W of step 0 (group 0), A of steps 0 and 1 (group 1)
        if (grp == 0) {
            pissue(0, lw0);
        } else {
            pissue(0, la0);
            if (nk > 1) pissue(1, la1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(bias[j]));
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * WN + j * 16 + 4 * hh;
            const f32x4 b = n < p.N ? bias[j] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[i][j] = b;
        }
        __syncthreads();
        if (grp == 1) __builtin_amdgcn_s_barrier();  // group 1 one slot behind
        // step j: A in buffer a_j, W in w_j; group 0 moves W of step j + 1
        // to wst, group 1 A of step j + 2 to ast
        auto pstep = [&](int j, const f16 *a_j, const f16 *w_j, uint32_t wst, uint32_t ast)
                         __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
            if (grp == 0) {
                if (j + 1 < nk) pissue(j + 1, wst);
            } else {
                if (j + 2 < nk) pissue(j + 2, ast);
            }
            pmem(a_j, w_j);
            __builtin_amdgcn_sched_barrier(0);
            if (grp == 1) {
                if (j + 2 < nk)
                    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            // the compute phase at raised wave priority: the SIMD's other wave,
            // in its memory phase, then yields the issue slots it contends for
            __builtin_amdgcn_s_setprio(1);
            pcomp(a_j);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            if (grp == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };
        // unrolled by six (A period 3, W period 2) so every LDS access names
        // its buffer statically
#pragma unroll 1
        for (int kt = 0; kt < nk; kt += 6) {
            pstep(kt, A0, W0, lw1, la2);
            if (kt + 1 >= nk) break;
            pstep(kt + 1, A1, W1, lw0, la0);
            if (kt + 2 >= nk) break;
            pstep(kt + 2, A2, W0, lw1, la1);
            if (kt + 3 >= nk) break;
            pstep(kt + 3, A0, W1, lw0, la2);
            if (kt + 4 >= nk) break;
            pstep(kt + 4, A1, W0, lw1, la0);
            if (kt + 5 >= nk) break;
            pstep(kt + 5, A2, W1, lw0, la1);
        }
        if (grp == 0) __builtin_amdgcn_s_barrier();  // match group 1's extra barrier
    } else {
    f16x8 af[TM], bf0[TN], bf1[TN];
    auto slice = [&](const f16x8 (&bfc)[TN], f16x8 (&bfn)[TN], const f16 *asrc, const f16 *wsrc, int kk)
                     __attribute__((always_inline)) {
        const f16 *as = asrc + (wm * WM + frow) * BK;
        const f16 *bs = wsrc + (wn * WN + frow) * BK;
        const int ch = ((kk * 4 + (lane >> 4)) ^ fsw) << 3;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bfc[j], af[i], acc[i][j], 0, 0, 0);
            if (i < TN) bfn[i] = *reinterpret_cast<const f16x8 *>(bs + i * 16 * BK + ch);
            af[i] = *reinterpret_cast<const f16x8 *>(as + i * 16 * BK + ch);
        }
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int i = TN; i < TM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    // A tiles rotate through three buffers and W tiles through two: at the
    // barrier of step kt the buffers of tile kt are free, and they receive
    // A of step kt + 3 and W of step kt + 2 (issued W first).  So an A
    // transfer has two steps to land and a W transfer one.  The wait before
    // the barrier needs tile kt + 1: its A went out a step before the W, and
    // each wave's transfers complete in issue order, so only the AG
    // transfers of A for step kt + 2 may still be outstanding.
    auto step = [&](int kt, const f16 *a_cur, const f16 *w_cur, const f16 *a_nxt, const f16 *w_nxt, uint32_t a_cur_lds,
                    uint32_t w_cur_lds) __attribute__((always_inline)) {
        slice(bf0, bf1, a_cur, w_cur, 1);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 2 < nk)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(AG) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 2 < nk) issueW(kt + 2, w_cur_lds);
        if (kt + 3 < nk) issueA(kt + 3, a_cur_lds);
        __builtin_amdgcn_sched_barrier(0);
        slice(bf1, bf0, a_nxt, w_nxt, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    const f16 *A0 = smem0, *A1 = smem1, *A2 = smemA2, *W0 = smem0 + ASZ, *W1 = smem1 + ASZ;
    issueW(0, lw0);
    issueA(0, la0);
    if (nk > 1 && wave < LW) {
        issueA(1, la1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(AG) : "memory");
    } else {
        // (a wave that issues no direct loads has only the bias loads out)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // the bias registers are valid from here: nothing reads them earlier
#pragma unroll
    for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(bias[j]));
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + 4 * hh;
        const f32x4 b = n < p.N ? bias[j] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][j] = b;
    }
    __syncthreads();
    if (nk > 1) issueW(1, lw1);
    if (nk > 2) issueA(2, la2);
    {
        const f16 *as = A0 + (wm * WM + frow) * BK;
        const f16 *bs = W0 + (wn * WN + frow) * BK;
        const int ch = ((lane >> 4) ^ fsw) << 3;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const f16x8 *>(as + i * 16 * BK + ch);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf0[j] = *reinterpret_cast<const f16x8 *>(bs + j * 16 * BK + ch);
    }
    // unrolled by six (A period 3, W period 2) so every LDS access names its
    // buffer statically
#pragma unroll 1
    for (int kt = 0; kt < nk; kt += 6) {
        step(kt, A0, W0, A1, W1, la0, lw0);
        if (kt + 1 >= nk) break;
        step(kt + 1, A1, W1, A2, W0, la1, lw1);
        if (kt + 2 >= nk) break;
        step(kt + 2, A2, W0, A0, W1, la2, lw0);
        if (kt + 3 >= nk) break;
        step(kt + 3, A0, W1, A1, W0, la0, lw1);
        if (kt + 4 >= nk) break;
        step(kt + 4, A1, W0, A2, W1, la1, lw0);
        if (kt + 5 >= nk) break;
        step(kt + 5, A2, W1, A0, W0, la2, lw1);
    }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Epilogue through LDS.  Written straight from the accumulator layout,
    // each store would cover 16 rows x 16 bytes; instead each wave stages one
    // 32-row x 64-column block at a time in a private LDS region (the k-step
    // buffers are free now) and reads it back row-major, so the global
    // writes are whole 128-byte (fp16) or 256-byte (fp32) row segments.  The
    // region is the wave's own, and LDS operations of one wave complete in
    // order, so the only barrier is the one that retires the k-step buffers.
    constexpr bool F32OUT = EPI == WENC_EPI_CONV2 || EPI == WENC_EPI_RESID;
    constexpr int RS = F32OUT ? 64 + 4 : 64 + 8;        // row stride, elements (16 bytes of padding)
    constexpr int REGION = 32 * RS * (F32OUT ? 4 : 2);  // bytes per wave
    static_assert(WN % 64 == 0 && WM % 32 == 0 && (NW / 2) * REGION <= STAGE * 2, "staging fits in one k-step buffer");
    __syncthreads();
    char *stg = reinterpret_cast<char *>(wave < NW / 2 ? smem0 : smem1) + (wave % (NW / 2)) * REGION;
    // stage the wave's 32-row block i2 of column group cg: lane holds row
    // 16 g + frow, columns 16 j + 4 hh .. +3 (GELU applied here for conv2)
    auto stage_f32 = [&](int cg, int i2) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int cl = j * 16 + 4 * hh;
                const int srow = 16 * g + frow;
                const f32x4 v = acc[2 * i2 + g][cg * 4 + j];
                f32x4 w = v;
                if constexpr (EPI == WENC_EPI_CONV2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = gelu_erf(v[e]);
                }
                *reinterpret_cast<f32x4 *>(stg + (srow * RS + cl) * 4) = w;
            }
    };
    if constexpr (F32OUT) {
        // fp32 outputs: out = staged value + addend, where the addend is the
        // residual (read-modify-write of C) or the position row.  A unit is
        // a half of a 32-row block: 16 lanes per 64-float row, 4 rows per
        // instruction, 4 instructions.  Each unit's addend loads are issued
        // two units ahead, so their latency overlaps the staging, adds and
        // stores of the units before.  The loads and stores are buffer
        // operations whose offset is past the range for rows at or beyond M
        // and columns at or beyond N (a load then reads zero, a store is
        // dropped), so no branch splits them and the compiler's waits count
        // exactly the loads a unit needs.  (With a branch per row it waited
        // for every outstanding load before each store: one full memory
        // round trip per unit, 8 per 128-row wave tile.)
        constexpr int UNITS = 2 * (WM / 32);
        const int c = lane & 15, rq = lane >> 4;
        // C from the tile's first row on: offsets stay far below 2^31
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<float *>(p.C) + int64_t(m0) * p.ldc, 0, 0x7fffffff, 0x00020000);
        const __amdgpu_buffer_rsrc_t rpos = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(EPI == WENC_EPI_CONV2 ? p.pos : static_cast<const float *>(p.C)), 0, 0x7fffffff,
            0x00020000);
#pragma unroll
        for (int cg = 0; cg < WN / 64; ++cg) {
            const int n = n0 + wn * WN + cg * 64 + c * 4;
            // byte offset in C of row m (tile-relative) and column n, or past the range
            auto c_off = [&](int m) __attribute__((always_inline)) {
                return (m < p.M && n < p.N) ? uint32_t(((m - m0) * p.ldc + n) * 4) : OOB;
            };
            f32x4 addv[3][4];
            auto load_unit = [&](int u, f32x4 (&add)[4]) __attribute__((always_inline)) {
                const int mr = m0 + wm * WM + (u >> 1) * 32;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int m = mr + ((u & 1) * 4 + it) * 4 + rq;
                    if constexpr (EPI == WENC_EPI_RESID) {
                        add[it] = __builtin_amdgcn_raw_buffer_load_b128(rc, c_off(m), 0, 0);
                    } else {
                        const uint32_t t = uint32_t(m) - divu(uint32_t(m), p.pos_div) * p.pos_div.d;
                        const uint32_t off = (m < p.M && n < p.N) ? uint32_t((int(t) * p.N + n) * 4) : OOB;
                        add[it] = __builtin_amdgcn_raw_buffer_load_b128(rpos, off, 0, 0);
                    }
                }
            };
            load_unit(0, addv[0]);
            if (UNITS > 1) load_unit(1, addv[1 % 3]);
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                if (u + 2 < UNITS) load_unit(u + 2, addv[(u + 2) % 3]);
                if ((u & 1) == 0) stage_f32(cg, u >> 1);
                const int mr = m0 + wm * WM + (u >> 1) * 32;
                const int h0 = (u & 1) * 4;
                f32x4 w[4];
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    w[it] = *reinterpret_cast<const f32x4 *>(stg + (((h0 + it) * 4 + rq) * RS + c * 4) * 4);
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    __builtin_amdgcn_raw_buffer_store_b128(w[it] + addv[u % 3][it], rc, c_off(mr + (h0 + it) * 4 + rq), 0,
                                                          0);
            }
        }
        return;
    }
    // GELU fp16 output: C from the tile's first row on (its batch item cb0, row cr0)
    const uint32_t cb0 = divu(uint32_t(m0), p.c_div), cr0 = uint32_t(m0) - cb0 * p.c_div.d;
#pragma unroll
    for (int cg = 0; cg < WN / 64; ++cg) {
        const int nw = n0 + wn * WN + cg * 64;  // first column of this 64-column group
        bool vtile = false;                     // QKV: the group is one head of v
        int vhead = 0;
        float sc = 1.0f;
        if constexpr (EPI == WENC_EPI_QKV) {
            const int slice = nw / p.dmodel;  // a 64-column group is one head of q, k or v
            vtile = slice == 2;
            vhead = (nw - 2 * p.dmodel) >> 6;
            sc = slice == 0 ? p.q_scale : 1.0f;
        }
#pragma unroll
        for (int i2 = 0; i2 < WM / 32; ++i2) {
            const int mr = m0 + wm * WM + i2 * 32;
            if (mr >= p.M) break;
            // stage: lane holds row 16 g + frow, columns 16 j + 4 hh .. +3
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const int cl = j * 16 + 4 * hh;
                    const int srow = 16 * g + frow;
                    const f32x4 v = acc[2 * i2 + g][cg * 4 + j];
                    f16x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (EPI == WENC_EPI_GELU_F16)
                            o[e] = (f16)gelu_erf(v[e]);
                        else
                            o[e] = (f16)(v[e] * sc);
                    }
                    *reinterpret_cast<f16x4 *>(stg + (srow * RS + cl) * 2) = o;
                }
            if (vtile) {
                if constexpr (EPI == WENC_EPI_QKV) {
                    // V^T [b][h][dim][slot]: the block's 32 rows are two 16-key
                    // groups of one batch item each (the row space is padded to a
                    // multiple of 16 keys).  A run is 8 consecutive slots of one
                    // dimension: slots 16 G + 8 s8 .. +7 hold keys 16 G +
                    // vt_slot(8 s8 + q) (the slot order is an involution).  Four
                    // consecutive lanes cover one dimension's 32 slots; keys at or
                    // past T are written as zeros.
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int run = it * 64 + lane;
                        const int s8 = run & 1, gr = (run >> 1) & 1, e = run >> 2;
                        const uint32_t mg = uint32_t(mr + 16 * gr);
                        const uint32_t bb = divu(mg, p.t_div);
                        const uint32_t t0 = mg - bb * p.t_div.d;
                        f16x8 o;
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const uint32_t key = vt_slot(uint32_t(8 * s8 + q));
                            const f16 val = *reinterpret_cast<const f16 *>(stg + ((16 * gr + key) * RS + e) * 2);
                            o[q] = t0 + key < uint32_t(p.T) ? val : (f16)0.0f;
                        }
                        if (int(mg) < p.M)
                            *reinterpret_cast<f16x8 *>(p.vt + ((int64_t(bb) * p.H + vhead) * 64 + e) * p.ldvt + t0 + 8 * s8) = o;
                    }
                    // the last key group of a batch item also clears slots
                    // t_div.d .. ldvt-1 of its 64 dimensions
#pragma unroll
                    for (int gr = 0; gr < 2; ++gr) {
                        const uint32_t mg = uint32_t(mr + 16 * gr);
                        const uint32_t bb = divu(mg, p.t_div);
                        const uint32_t t0 = mg - bb * p.t_div.d;
                        if (int(mg) < p.M && t0 + 16 == p.t_div.d) {
                            const int nz = (p.ldvt - int(p.t_div.d)) / 8;
                            for (int run = lane; run < nz * 64; run += 64) {
                                const int e = run & 63, zc = run >> 6;
                                *reinterpret_cast<f16x8 *>(p.vt + ((int64_t(bb) * p.H + vhead) * 64 + e) * p.ldvt +
                                                           p.t_div.d + 8 * zc) = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
                            }
                        }
                    }
                }
            } else {
                // 8 lanes per 64-half row, 8 rows per instruction
                const int c = lane & 7, r8 = lane >> 3;
                const int n = nw + c * 8;
                bool stored = false;
                if constexpr (EPI == WENC_EPI_GELU_F16) {
                    if (p.c_run8) {
                        const __amdgpu_buffer_rsrc_t rcg = __builtin_amdgcn_make_buffer_rsrc(
                            static_cast<f16 *>(p.C) + int64_t(cb0) * p.c_bs + (int64_t(cr0) + p.c_off) * p.ldc, 0,
                            0x7fffffff, 0x00020000);
                        // All four rows read back first, then four buffer
                        // stores whose offset is past the range for rows at or
                        // beyond M and columns at or beyond N (the store is
                        // dropped): no branch around a store, no 64-bit address
                        // arithmetic per row, offsets from the tile's first row.
                        f16x8 o[4];
#pragma unroll
                        for (int it = 0; it < 4; ++it)
                            o[it] = *reinterpret_cast<const f16x8 *>(stg + ((it * 8 + r8) * RS + c * 8) * 2);
#pragma unroll
                        for (int it = 0; it < 4; ++it) {
                            const int m = mr + it * 8 + r8;
                            const uint32_t bi = divu(uint32_t(m), p.c_div);
                            const int64_t e = int64_t(bi - cb0) * p.c_bs +
                                              (int64_t(uint32_t(m) - bi * p.c_div.d) - int64_t(cr0)) * p.ldc + n;
                            const uint32_t off = (m < p.M && n < p.N) ? uint32_t(e * 2) : OOB;
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o[it]), rcg, off, 0, 0);
                        }
                        stored = true;
                    }
                }
                if constexpr (EPI == WENC_EPI_QKV) {
                    if (p.qk_run8) {
                        // q or k of head hq, [b][h][t][64]: key t of batch item b
                        // is 128 bytes at ((b H + hq) T + t) 64; a pad row (t at
                        // or past T) or a row at or past M gets an out-of-range
                        // offset, so the store is dropped
                        const int sl = nw / p.dmodel, hq = (nw - sl * p.dmodel) >> 6;
                        const uint32_t qb0 = divu(uint32_t(m0), p.t_div), qt0 = uint32_t(m0) - qb0 * p.t_div.d;
                        const __amdgpu_buffer_rsrc_t rqk = __builtin_amdgcn_make_buffer_rsrc(
                            (sl == 0 ? p.q : p.k) + ((int64_t(qb0) * p.H + hq) * p.T + qt0) * 64, 0, 0x7fffffff, 0x00020000);
                        f16x8 o[4];
#pragma unroll
                        for (int it = 0; it < 4; ++it)
                            o[it] = *reinterpret_cast<const f16x8 *>(stg + ((it * 8 + r8) * RS + c * 8) * 2);
#pragma unroll
                        for (int it = 0; it < 4; ++it) {
                            const int m = mr + it * 8 + r8;
                            const uint32_t bb = divu(uint32_t(m), p.t_div), t = uint32_t(m) - bb * p.t_div.d;
                            const int64_t e = (int64_t(bb - qb0) * p.H * p.T + (int64_t(t) - int64_t(qt0))) * 64 + c * 8;
                            const uint32_t off = (m < p.M && t < uint32_t(p.T) && n < p.N) ? uint32_t(e * 2) : OOB;
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o[it]), rqk, off, 0, 0);
                        }
                        stored = true;
                    }
                }
                if (!stored) {
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int r = it * 8 + r8;
                        const f16x8 o = *reinterpret_cast<const f16x8 *>(stg + (r * RS + c * 8) * 2);
                        const int m = mr + r;
                        if (m < p.M && n < p.N) epi_row8<EPI>(p, m, n, o);
                    }
                }
            }
        }
    }
}

// Tile configuration shared by every launch in the process (a test-only
// override): tile 0 = 128x128 x 4 waves, 1 = 256x256 x 8 waves, 2 = 256x256
// x 8 waves with the lockstep main loop instead of the ping-pong one,
// anything else = chosen per launch; split 0 keeps a launch on one tile size.  The
// environment (WENC_GEMM_TILE, WENC_GEMM_SPLIT) is read once, under the
// thread-safe initialisation of a function-local static; later changes go
// through gemm_mode.  Atomics, so launches on other threads read a whole
// value.
struct TileMode {
    std::atomic<int> tile, split;
    TileMode() {
        const char *e = std::getenv("WENC_GEMM_TILE");
        const char *f = std::getenv("WENC_GEMM_SPLIT");
        tile.store(e ? std::atoi(e) : 99);
        split.store(f ? std::atoi(f) : 1);
    }
};

TileMode &tile_mode() {
    static TileMode m;
    return m;
}

template <int BM, int BN, int WM, int WN, int NW, int TAG, int PP>
hipError_t launch_cfg(const GemmP &base, int epi, hipStream_t s) {
    GemmP p = base;
    p.tiles_m = (p.M - p.m_begin + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    const dim3 grid(p.tiles_m * p.tiles_n), block(NW * 64);
    switch (epi) {
        case WENC_EPI_GELU_F16: gemm_kernel<BM, BN, WM, WN, NW, WENC_EPI_GELU_F16, TAG, PP><<<grid, block, 0, s>>>(p); break;
        case WENC_EPI_CONV2: gemm_kernel<BM, BN, WM, WN, NW, WENC_EPI_CONV2, 0, PP><<<grid, block, 0, s>>>(p); break;
        case WENC_EPI_RESID: gemm_kernel<BM, BN, WM, WN, NW, WENC_EPI_RESID, TAG, PP><<<grid, block, 0, s>>>(p); break;
        case WENC_EPI_QKV: gemm_kernel<BM, BN, WM, WN, NW, WENC_EPI_QKV, 0, PP><<<grid, block, 0, s>>>(p); break;
        case WENC_EPI_KV: gemm_kernel<BM, BN, WM, WN, NW, WENC_EPI_KV, 0, PP><<<grid, block, 0, s>>>(p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The 256 x 256 kernel runs the ping-pong main loop unless `lockstep`.
template <int BM, int BN, int WM, int WN, int NW>
hipError_t launch_tagged(const GemmP &p, int epi, int tag, hipStream_t s, bool lockstep = false) {
    if constexpr (BM == 256) {
        if (!lockstep)
            return tag ? launch_cfg<BM, BN, WM, WN, NW, 1, 1>(p, epi, s) : launch_cfg<BM, BN, WM, WN, NW, 0, 1>(p, epi, s);
    }
    return tag ? launch_cfg<BM, BN, WM, WN, NW, 1, 0>(p, epi, s) : launch_cfg<BM, BN, WM, WN, NW, 0, 0>(p, epi, s);
}


}  // namespace

// Compute units of the current device (cached per device; a race only
// stores the same value twice).
long cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int gemm_mode(int tile, int split) {
    if (tile < -1 || tile > 2 || split < 0 || split > 1) return -1;
    if (tile == -1) {
        const char *e = std::getenv("WENC_GEMM_TILE");
        tile = e ? std::atoi(e) : 99;
    }
    tile_mode().tile.store(tile);
    tile_mode().split.store(split);
    return 0;
}

const char *gemm_check(const wenc_gemm_args &a) {
    if (!a.A || !a.W || !a.bias) return "gemm: A, W and bias must be non-null";
    if (a.M < 0 || a.N <= 0 || a.K <= 0) return "gemm: need M >= 0, N > 0, K > 0";
    if (a.K % 8 || a.lda % 8 || a.ldw % 8 || a.a_batch_stride % 8)
        return "gemm: K, lda, ldw and a_batch_stride must be multiples of 8 (16-byte rows)";
    if (a.N % 4 || a.ldc % 4 || a.c_batch_stride % 4)
        return "gemm: N, ldc and c_batch_stride must be multiples of 4 (vector stores)";
    if (a.ldw < a.K) return "gemm: ldw < K";
    if (a.a_rows_per_batch <= 0 || a.a_rows_per_batch >= (1 << 16)) return "gemm: a_rows_per_batch out of [1, 65535]";
    if (a.M >= (1 << 24)) return "gemm: M must be < 2^24";
    // per-tile buffer offsets are 31-bit: a 256-row tile of A (which may
    // straddle two batch items) and of W must span well under 2 GiB
    if (int64_t(a.lda) * 256 * 2 + int64_t(a.a_batch_stride) * 2 >= (int64_t(1) << 30) ||
        int64_t(a.ldw) * 256 * 2 >= (int64_t(1) << 30))
        return "gemm: operand rows too long for 31-bit tile offsets";
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
            if (int64_t(a.pos_rows) * a.N * 4 >= (int64_t(1) << 31)) return "gemm: position table too large for 31-bit offsets";
            if (int64_t(a.ldc) * 256 * 4 >= (int64_t(1) << 30)) return "gemm: C rows too long for 31-bit tile offsets";
            break;
        case WENC_EPI_RESID:
            if (!a.C) return "gemm: C is null";
            if (a.ldc < a.N) return "gemm: ldc < N";
            if (int64_t(a.ldc) * 256 * 4 >= (int64_t(1) << 30)) return "gemm: C rows too long for 31-bit tile offsets";
            break;
        case WENC_EPI_QKV:
            if (!a.q || !a.k || !a.vt) return "gemm: q, k, vt must be non-null";
            if (a.n_head <= 0 || a.N != 3 * 64 * a.n_head) return "gemm: QKV needs N == 3 * 64 * n_head";
            if (a.T <= 0 || a.T >= (1 << 16) || a.M % a.T) return "gemm: QKV needs 0 < T < 65536 and M % T == 0";
            if (a.ldvt < a.T || a.ldvt % 64) return "gemm: ldvt must be a multiple of 64 and >= T";
            if (!(a.a_rows_per_batch >= a.M || a.a_batch_stride == int64_t(a.a_rows_per_batch) * a.lda))
                return "gemm: QKV needs row-linear A (row m at m * lda)";
            if (int64_t(a.M / a.T) * ((a.T + 15) & ~15) >= (1 << 24)) return "gemm: QKV rows padded to 16 keys must be < 2^24";
            break;
        case WENC_EPI_KV:
            if (!a.C) return "gemm: C is null";
            if (a.n_split <= 0 || a.n_split > a.N || a.n_split % 4) return "gemm: KV needs 0 < n_split <= N, n_split % 4 == 0";
            if (a.n_split < a.N && !a.C2) return "gemm: C2 is null";
            if (a.ldc < a.n_split || a.ldc < a.N - a.n_split) return "gemm: ldc < max(n_split, N - n_split)";
            break;
        default:
            return "gemm: unknown epilogue";
    }
    return nullptr;
}

hipError_t launch_gemm(const wenc_gemm_args &a, hipStream_t s, int tag, int cu_div) {
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
    if (a.epilogue == WENC_EPI_GELU_F16) {
        // a row's offset from its tile's first row is non-negative when batch
        // items do not overlap, and below 2 GiB when a tile's 256 rows (which
        // span at most 256 / D + 2 items of D rows) stay within it
        const int64_t D = a.c_rows_per_batch;
        const bool ordered = D >= a.M || a.c_batch_stride >= D * a.ldc;
        const int64_t span = (256 / D + 2) * a.c_batch_stride + (256 + int64_t(a.c_row_offset)) * a.ldc + a.N;
        p.c_run8 = a.N % 8 == 0 && a.c_row_offset >= 0 && ordered && span * 2 < (int64_t(1) << 31);
    }
    p.pos = a.pos;
    p.pos_div = make_divu(a.pos_rows > 0 ? a.pos_rows : 1);
    p.q = reinterpret_cast<f16 *>(a.q);
    p.k = reinterpret_cast<f16 *>(a.k);
    p.vt = reinterpret_cast<f16 *>(a.vt);
    p.C2 = reinterpret_cast<f16 *>(a.C2);
    p.n_split = a.n_split;
    p.t_div = make_divu(a.T > 0 ? a.T : 1);
    p.H = a.n_head;
    p.ldvt = a.ldvt;
    p.dmodel = a.n_head * 64;
    p.q_scale = a.q_scale;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.a_valid = 1 << 30;
    p.T = a.T;
    if (a.epilogue == WENC_EPI_QKV) {
        // Rows are padded to a multiple of 16 keys per batch item, so that a
        // 16-row block of the tile is one V^T slot group; pad rows read zero
        // (row-linear A, checked by gemm_check) and are not stored.
        const int tp = (a.T + 15) & ~15;
        p.M = (a.M / a.T) * tp;
        p.a_div = make_divu(tp);
        p.a_bs = int64_t(a.T) * a.lda;
        p.a_valid = a.T;
        p.t_div = make_divu(tp);
        // a tile's 256 rows span at most 256 / tp + 2 batch items of H T keys of 64
        p.qk_run8 = (int64_t(256 / tp + 2) * a.n_head * a.T + 256) * 64 * 2 < (int64_t(1) << 31);
    }
    const int tile = tile_mode().tile.load(), split = tile_mode().split.load();
    const bool lockstep = tile == 2;
    const int plan_tile = tile == 0 || tile == 1 ? tile : (lockstep ? 1 : -1);
    const GemmPlan plan = gemm_plan(p.M, p.N, cu_count(), plan_tile, split, std::max(cu_div, 1));
    if (plan.kind == GEMM_PLAN_SMALL) return launch_tagged<128, 128, 64, 64, 4>(p, a.epilogue, tag, s);
    if (plan.kind == GEMM_PLAN_BIG) return launch_tagged<256, 256, 128, 64, 8>(p, a.epilogue, tag, s, lockstep);
    GemmP big = p;
    big.M = plan.big_rows;
    const hipError_t e = launch_tagged<256, 256, 128, 64, 8>(big, a.epilogue, tag, s, lockstep);
    if (e != hipSuccess) return e;
    GemmP tail = p;
    tail.m_begin = plan.big_rows;
    return launch_tagged<128, 128, 64, 64, 4>(tail, a.epilogue, tag, s);
}

GemmPlan gemm_plan(int M, int N, long cus, int tile, int split, int streams) {
    if (tile == 1) return {GEMM_PLAN_BIG, M};
    if (tile == 0) return {GEMM_PLAN_SMALL, 0};
    const long tn_big = (N + 255) / 256, tm_big = (long(M) + 255) / 256;
    if (streams > 1) {
        // Launches of a forward split over several streams run side by side,
        // each with about cus / streams compute units: the 256 x 256 tiles
        // from 0.75 tiles per such unit on, on whole launches (measured on
        // two streams: on c3's 24000-row projections, whose halves have 141
        // such tiles at N = 768, they beat 128 x 128 tiles by 7% of a
        // step; carving the last tile rows into small tiles, which pays on
        // one stream, cost 1-7%).
        const long share = std::max(1L, cus / streams);
        return 4 * tm_big * tn_big < 3 * share ? GemmPlan{GEMM_PLAN_SMALL, 0} : GemmPlan{GEMM_PLAN_BIG, M};
    }
    // 256 x 256 tiles when they fill the CUs at least 1.75 times over
    // (measured on 256 CUs: on 24000 x 768 x {768, 3072}, 282 such tiles,
    // the 128 x 128 tiles at two workgroups per CU are 10-20% faster).
    if (4 * tm_big * tn_big < 7 * cus) return {GEMM_PLAN_SMALL, 0};
    // The 256 x 256 kernel runs one tile per CU at a time, so a tile count
    // just past a multiple of the CU count leaves most CUs idle in the last
    // round.  Then the last tile rows go to the 128 x 128 kernel instead (two
    // workgroups per CU), whose round costs about 0.6 of a big round; both
    // kernels sum each output over k in the same order, so the split changes
    // no result bit.  R = the number of 256-row tile rows kept big.
    long best_r = tm_big;
    if (split) {
        auto rounds = [](long n, long per) { return double((n + per - 1) / per); };
        double best = rounds(tm_big * tn_big, cus);
        for (long r = tm_big - 1; r >= 1 && r >= tm_big - 64; --r) {
            const long small = ((M - 256 * r + 127) / 128) * ((N + 127) / 128);
            const double cost = rounds(r * tn_big, cus) + 0.6 * rounds(small, 2 * cus);
            if (cost < best - 0.05) {
                best = cost;
                best_r = r;
            }
        }
    }
    if (best_r == tm_big) return {GEMM_PLAN_BIG, M};
    return {GEMM_PLAN_SPLIT, int(256 * best_r)};
}

}  // namespace wk
