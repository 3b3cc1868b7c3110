// Host runtime of libwenc.so: the C ABI declared in include/wenc.h.
//
// Owns one device arena for the repacked weights (one upload per load, as
// the whisper README's memory notes describe: the checkpoint is mapped,
// uploaded once and released) and one arena for the activations of
// max_batch windows.  wenc_forward only enqueues kernels on the caller's
// stream: ingest, conv1, conv2, then per block LN1, QKV, attention,
// out_proj, LN2, fc1, fc2, and the final LN (3 + 7 L + 1 launches per chunk).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"
#include "wenc.h"

namespace {

// Message of the last failure in this thread (a fixed buffer: reporting a
// failure of a handle-less call allocates nothing).
thread_local char g_err[512];

int fail(std::string *dst, int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    if (dst) *dst = g_err;
    return code;
}

// IEEE binary16 -> binary32, exact (subnormals, infinities and NaN included).
float half_to_float(uint16_t h) {
    const uint32_t sign = uint32_t(h & 0x8000u) << 16;
    uint32_t exp = (h >> 10) & 0x1f;
    uint32_t man = h & 0x3ffu;
    uint32_t bits;
    if (exp == 0) {
        if (man == 0) {
            bits = sign;
        } else {
            exp = 127 - 15 + 1;
            while (!(man & 0x400u)) {
                man <<= 1;
                --exp;
            }
            man &= 0x3ffu;
            bits = sign | (exp << 23) | (man << 13);
        }
    } else if (exp == 31) {
        bits = sign | 0x7f800000u | (man << 13);
    } else {
        bits = sign | ((exp + 127 - 15) << 23) | (man << 13);
    }
    float f;
    std::memcpy(&f, &bits, 4);
    return f;
}

struct Bump {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = (off + 255) & ~size_t(255);
        off = o + bytes;
        return o;
    }
};

struct LayerOff {
    size_t ln1_g, ln1_b, wqkv, bqkv, wo, bo, ln2_g, ln2_b, fc1_w, fc1_b, fc2_w, fc2_b;
};

struct WeightLayout {
    size_t conv1_w, conv1_b, conv2_w, conv2_b, pos, lnf_g, lnf_b;
    std::vector<LayerOff> layers;
    size_t total;
};

WeightLayout weight_layout(const wenc_config &c) {
    const size_t d = c.d_model, F = c.d_ff, nm = c.n_mels, T = c.n_ctx;
    WeightLayout w;
    Bump b;
    w.conv1_w = b.take(2 * d * 3 * nm);
    w.conv1_b = b.take(4 * d);
    w.conv2_w = b.take(2 * d * 3 * d);
    w.conv2_b = b.take(4 * d);
    w.pos = b.take(4 * T * d);
    for (int l = 0; l < c.n_layer; ++l) {
        LayerOff o;
        o.ln1_g = b.take(4 * d);
        o.ln1_b = b.take(4 * d);
        o.wqkv = b.take(2 * 3 * d * d);
        o.bqkv = b.take(4 * 3 * d);
        o.wo = b.take(2 * d * d);
        o.bo = b.take(4 * d);
        o.ln2_g = b.take(4 * d);
        o.ln2_b = b.take(4 * d);
        o.fc1_w = b.take(2 * F * d);
        o.fc1_b = b.take(4 * F);
        o.fc2_w = b.take(2 * d * F);
        o.fc2_b = b.take(4 * d);
        w.layers.push_back(o);
    }
    w.lnf_g = b.take(4 * d);
    w.lnf_b = b.take(4 * d);
    w.total = (b.off + 255) & ~size_t(255);
    return w;
}

struct ScratchLayout {
    size_t melp, c1, x, xn, q, k, vt, ao, hbuf, total;
    int ldvt;
};

ScratchLayout scratch_layout(const wenc_config &c) {
    const size_t B = c.max_batch, F = c.n_frames, nm = c.n_mels, d = c.d_model, T = c.n_ctx, H = c.n_head,
                 Fd = c.d_ff;
    ScratchLayout s;
    s.ldvt = int((T + 63) / 64 * 64);
    Bump b;
    s.melp = b.take(2 * B * (F + 2) * nm);
    s.c1 = b.take(2 * B * (F + 2) * d);
    s.x = b.take(4 * B * T * d);
    s.xn = b.take(2 * B * T * d);
    s.q = b.take(2 * B * H * T * 64);
    s.k = b.take(2 * B * H * T * 64);
    s.vt = b.take(2 * B * H * 64 * size_t(s.ldvt));
    s.ao = b.take(2 * B * T * d);
    s.hbuf = b.take(2 * B * T * Fd);
    s.total = (b.off + 255) & ~size_t(255);
    return s;
}

const char *config_error(const wenc_config *c) {
    if (!c) return "config is NULL";
    if (c->head_dim != 64) return "head_dim must be 64";
    if (c->n_head <= 0 || c->d_model != c->n_head * 64) return "d_model must equal n_head * 64 with n_head > 0";
    if (c->d_model > 2048) return "d_model must be <= 2048";
    if (c->n_mels <= 0 || c->n_mels % 8 || c->n_mels > 4096) return "n_mels must be a positive multiple of 8, <= 4096";
    if (c->d_ff <= 0 || c->d_ff % 8 || c->d_ff > 65536) return "d_ff must be a positive multiple of 8, <= 65536";
    if (c->n_layer < 0 || c->n_layer > 4096) return "n_layer must be in [0, 4096]";
    if (c->n_ctx <= 0 || c->n_ctx >= 32768 || c->n_frames != 2 * c->n_ctx)
        return "n_frames must equal 2 * n_ctx with 0 < n_ctx < 32768";
    if (!(c->ln_eps > 0.f) || !std::isfinite(c->ln_eps)) return "ln_eps must be positive and finite";
    if (c->final_ln != 0 && c->final_ln != 1) return "final_ln must be 0 or 1";
    if (c->max_batch < 1) return "max_batch must be >= 1";
    if (int64_t(c->max_batch) * c->n_frames >= (int64_t(1) << 24)) return "max_batch * n_frames must be < 2^24";
    return nullptr;
}

size_t blob_halves(const wenc_config &c) {
    const size_t d = c.d_model, F = c.d_ff, nm = c.n_mels, T = c.n_ctx;
    const size_t layer = 2 * d + 4 * d * d + 2 * d + d + 2 * d + F * d + F + d * F + d;
    return d * nm * 3 + d + d * d * 3 + d + T * d + c.n_layer * layer + 2 * d;
}

// Slaney's auditory-toolbox mel scale: linear (200/3 Hz per mel) below 1 kHz,
// logarithmic above (27 mels per factor 6.4).
double hz_to_mel_slaney(double f) { return f < 1000.0 ? f / (200.0 / 3.0) : 15.0 + std::log(f / 1000.0) / (std::log(6.4) / 27.0); }
double mel_to_hz_slaney(double m) { return m < 15.0 ? m * (200.0 / 3.0) : 1000.0 * std::exp((std::log(6.4) / 27.0) * (m - 15.0)); }

// Constant tables of the log-mel frontend (CKE page, "The Frontend"), in fp64
// rounded to fp32: (cos, -sin) of 2 pi i / 400; the periodic Hann window
// 0.5 - 0.5 cos(2 pi i / 400); and n_mels triangles whose corners are
// evenly spaced in Slaney mels from 0 Hz to 8 kHz, each scaled by 2 / (its
// width in Hz) (unit area), sampled at the 201 bins k * 40 Hz.  Filter m is
// kept as a window of 16 nch bins from mstart[m] that holds every non-zero
// weight (nch the same for all filters, the window inside bins 0 .. 200):
// mwt[m][i] is the weight of bin mstart[m] + i, zero outside the triangle.
struct FrontendTables {
    std::vector<float> tab, win, mwt;
    std::vector<int32_t> mstart;
    int nch = 1;
};

FrontendTables frontend_tables(int n_mels) {
    FrontendTables t;
    const double pi = 3.14159265358979323846;
    t.tab.resize(800);
    t.win.resize(400);
    for (int i = 0; i < 400; ++i) {
        const double a = 2.0 * pi * i / 400.0;
        t.tab[2 * i] = float(std::cos(a));
        t.tab[2 * i + 1] = float(-std::sin(a));
        t.win[i] = float(0.5 - 0.5 * std::cos(a));
    }
    const double top = hz_to_mel_slaney(8000.0);
    std::vector<double> c(n_mels + 2);
    for (int i = 0; i < n_mels + 2; ++i) c[i] = mel_to_hz_slaney(top * i / (n_mels + 1));
    std::vector<float> dense(size_t(n_mels) * 201);
    std::vector<int> first(n_mels, -1), last(n_mels, -1);
    for (int i = 0; i < n_mels; ++i)
        for (int k = 0; k <= 200; ++k) {
            const double hz = 40.0 * k;
            const double rise = (hz - c[i]) / (c[i + 1] - c[i]);
            const double fall = (c[i + 2] - hz) / (c[i + 2] - c[i + 1]);
            const float w = float(std::max(0.0, std::min(rise, fall)) * 2.0 / (c[i + 2] - c[i]));
            dense[size_t(i) * 201 + k] = w;
            if (w != 0.0f) {
                if (first[i] < 0) first[i] = k;
                last[i] = k;
            }
        }
    for (int i = 0; i < n_mels; ++i)
        if (first[i] >= 0) t.nch = std::max(t.nch, (last[i] - first[i] + 16) / 16);
    const int width = 16 * t.nch;
    t.mstart.assign(n_mels, 0);
    t.mwt.assign(size_t(n_mels) * width, 0.0f);
    for (int i = 0; i < n_mels; ++i) {
        if (first[i] < 0) continue;  // an empty triangle: all weights zero
        const int s = std::max(0, std::min(first[i], 201 - width));
        t.mstart[i] = s;
        for (int k = first[i]; k <= last[i]; ++k) t.mwt[size_t(i) * width + (k - s)] = dense[size_t(i) * 201 + k];
    }
    return t;
}

// True when p is not a multiple of `align` bytes (the kernels' vector
// loads and stores need 16-byte aligned fp32 rows).
bool misaligned(const void *p, uintptr_t align) { return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0; }

struct ProfRec {
    int site;
    hipEvent_t e0, e1;
};

}  // namespace

struct wenc {
    wenc_config cfg;
    int device = 0;
    char *warena = nullptr;
    char *sarena = nullptr;
    char *xarena = nullptr;  // cross-attention K/V weights (wenc_load_cross)
    char *farena = nullptr;  // log-mel tables and per-tile maxima (when n_mels suits the frontend)
    size_t f_win = 0, f_mwt = 0, f_mstart = 0, f_blk = 0;
    int f_nch = 1;  // 16-bin windows per mel filter in the log-mel tables
    int n_dec = 0;
    size_t x_stride = 0;     // bytes per decoder layer in xarena: W_kv fp16 [2d][d], then bias fp32 [2d]
    WeightLayout wl;
    ScratchLayout sl;
    bool loaded = false;
    bool debug_sync = false;
    std::string err;
    uint32_t prof_mask = 0;
    std::vector<ProfRec> prof_pending;
    std::vector<hipEvent_t> event_pool;
    // Streams of a split forward beside the caller's, with the events that
    // fork them from it and join them back (created with the handle, at the
    // default priority).
    static constexpr int MAX_PARTS = 4;
    hipStream_t aux[MAX_PARTS - 1] = {};
    hipEvent_t ev_fork = nullptr, ev_join[MAX_PARTS - 1] = {};
    int n_parts = 2;  // a chunk's windows are split over this many streams
    // Recorded forward (wenc_forward_graph): the graph of one forward over
    // (g_mel, g_out, g_batch, g_nctx), recorded on the capture stream.
    hipStream_t cap = nullptr;
    hipGraphExec_t gexec = nullptr;
    const float *g_mel = nullptr;
    float *g_out = nullptr;
    int g_batch = 0, g_nctx = 0;

    template <class T>
    T *W(size_t off) const { return reinterpret_cast<T *>(warena + off); }
    template <class T>
    T *S(size_t off) const { return reinterpret_cast<T *>(sarena + off); }

    hipEvent_t take_event() {
        if (!event_pool.empty()) {
            hipEvent_t e = event_pool.back();
            event_pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }

    // Launch one site, optionally bracketed by timing events.
    template <class Fn>
    int site(int s, hipStream_t st, Fn &&launch) {
        hipEvent_t e0 = nullptr, e1 = nullptr;
        const bool prof = (prof_mask >> s) & 1u;
        if (prof) {
            e0 = take_event();
            e1 = take_event();
            if (!e0 || !e1) return fail(&err, WENC_EHIP, "hipEventCreate failed");
            const hipError_t er = hipEventRecord(e0, st);
            if (er != hipSuccess) return fail(&err, WENC_EHIP, "hipEventRecord: %s", hipGetErrorString(er));
        }
        hipError_t e = launch();
        if (prof) {
            const hipError_t er = hipEventRecord(e1, st);
            prof_pending.push_back({s, e0, e1});
            if (er != hipSuccess) return fail(&err, WENC_EHIP, "hipEventRecord: %s", hipGetErrorString(er));
        }
        if (e != hipSuccess) return fail(&err, WENC_EHIP, "launch at site %d failed: %s", s, hipGetErrorString(e));
        if (debug_sync) {
            e = hipStreamSynchronize(st);
            if (e == hipSuccess) e = hipGetLastError();
            if (e != hipSuccess) return fail(&err, WENC_EHIP, "site %d failed at sync: %s", s, hipGetErrorString(e));
        }
        return WENC_OK;
    }

    int forward_chunk(const float *mel, int nb, int T, float *out, hipStream_t st, int tap, void *tap_dst);
    int forward_part(const float *mel, int b0, int nb, int T, float *out, hipStream_t st, int cu_div, int tap,
                     void *tap_dst);
    int chunk_cap(int T) const;
};

#define WENC_TRY(expr)                 \
    do {                               \
        const int rc_ = (expr);        \
        if (rc_ != WENC_OK) return rc_; \
    } while (0)

// Windows of T positions (2T frames) one pass through the scratch can hold.
// The buffers are sized for max_batch windows of the configured n_ctx and
// packed densely at any T <= n_ctx, so a shortened context fits more windows.
int wenc::chunk_cap(int T) const {
    const int64_t B = cfg.max_batch, Tc = cfg.n_ctx, Fc = cfg.n_frames, F = 2 * int64_t(T);
    const int64_t ldvt = (T + 63) / 64 * 64;
    int64_t cap = std::min({B * Tc / T, B * (Fc + 2) / (F + 2), B * sl.ldvt / ldvt});
    cap = std::min(cap, ((int64_t(1) << 24) - 1) / F);  // row indices of the conv GEMMs stay < 2^24
    return int(std::max<int64_t>(cap, 1));
}

// One chunk of nb windows (mel [nb][2T][n_mels] -> out [nb][T][d]).  Unless
// a tap is asked for, the windows are split into n_parts groups that each
// run the whole path on a stream of their own: the first group on the
// caller's stream, the others on the handle's streams, forked from the
// caller's stream with an event and joined back before the call returns.
// The groups use disjoint window slices of the scratch.  Their kernels
// share the device, so one group's LayerNorms, residual epilogues and last
// partial round of tiles overlap another group's work, and every output is
// computed exactly as in one launch over all windows: windows are
// independent, and no kernel's per-element arithmetic depends on the batch.
int wenc::forward_chunk(const float *mel, int nb, int T, float *out, hipStream_t st, int tap, void *tap_dst) {
    const int parts = tap >= 0 ? 1 : std::max(1, std::min(n_parts, nb));
    if (parts == 1) return forward_part(mel, 0, nb, T, out, st, 1, tap, tap_dst);
    const size_t F = 2 * size_t(T);
    hipError_t e = hipEventRecord(ev_fork, st);
    for (int i = 0; i + 1 < parts && e == hipSuccess; ++i) e = hipStreamWaitEvent(aux[i], ev_fork, 0);
    if (e != hipSuccess) return fail(&err, WENC_EHIP, "forward: stream fork: %s", hipGetErrorString(e));
    int rc = WENC_OK, joined = 0;
    for (int i = 0; i < parts; ++i) {
        const int b0 = int(int64_t(nb) * i / parts), b1 = int(int64_t(nb) * (i + 1) / parts);
        hipStream_t si = i == 0 ? st : aux[i - 1];
        rc = forward_part(mel + size_t(b0) * F * cfg.n_mels, b0, b1 - b0, T, out + size_t(b0) * T * cfg.d_model, si,
                          parts, -1, nullptr);
        if (i > 0) ++joined;
        if (rc != WENC_OK) break;
    }
    // join every stream that received work, also after a failure, so the
    // caller's stream never runs ahead of work enqueued on the others
    for (int i = 0; i < joined; ++i) {
        hipError_t ej = hipEventRecord(ev_join[i], aux[i]);
        if (ej == hipSuccess) ej = hipStreamWaitEvent(st, ev_join[i], 0);
        if (ej != hipSuccess && e == hipSuccess) e = ej;
    }
    if (rc != WENC_OK) return rc;
    if (e != hipSuccess) return fail(&err, WENC_EHIP, "forward: stream join: %s", hipGetErrorString(e));
    return WENC_OK;
}

// Windows [b0, b0 + nb) of the chunk, on stream st, with the GEMM tile plan
// made for cus / cu_div compute units (the share one stream of a pipelined
// chunk can expect).
int wenc::forward_part(const float *mel, int b0, int nb, int T, float *out, hipStream_t st, int cu_div, int tap,
                       void *tap_dst) {
    const wenc_config &c = cfg;
    const int F = 2 * T, nm = c.n_mels, d = c.d_model, H = c.n_head, Fd = c.d_ff;
    const int M = nb * T;
    const int ldvt = (T + 63) / 64 * 64;
    const size_t wb = size_t(b0);  // window offset into the densely packed scratch
    uint16_t *melp = S<uint16_t>(sl.melp) + wb * (F + 2) * nm, *c1 = S<uint16_t>(sl.c1) + wb * (F + 2) * d;
    uint16_t *xn = S<uint16_t>(sl.xn) + wb * T * d;
    uint16_t *q = S<uint16_t>(sl.q) + wb * H * T * 64, *k = S<uint16_t>(sl.k) + wb * H * T * 64;
    uint16_t *vt = S<uint16_t>(sl.vt) + wb * H * 64 * ldvt;
    uint16_t *ao = S<uint16_t>(sl.ao) + wb * T * d, *hb = S<uint16_t>(sl.hbuf) + wb * T * Fd;
    float *x = S<float>(sl.x) + wb * T * d;

    WENC_TRY(site(WENC_SITE_INGEST, st, [&] { return wk::launch_ingest(mel, melp, c1, nb, F, nm, d, st); }));

    wenc_gemm_args g{};
    // conv1: output frame t reads padded frames t .. t+2 (3 n_mels contiguous values).
    g.A = melp;
    g.a_batch_stride = int64_t(F + 2) * nm;
    g.a_rows_per_batch = F;
    g.lda = nm;
    g.W = W<uint16_t>(wl.conv1_w);
    g.ldw = 3 * nm;
    g.bias = W<float>(wl.conv1_b);
    g.C = c1;
    g.c_batch_stride = int64_t(F + 2) * d;
    g.c_rows_per_batch = F;
    g.c_row_offset = 1;
    g.ldc = d;
    g.M = nb * F;
    g.N = d;
    g.K = 3 * nm;
    g.epilogue = WENC_EPI_GELU_F16;
    WENC_TRY(site(WENC_SITE_CONV1, st, [&] { return wk::launch_gemm(g, st, 0, cu_div); }));
    if (tap == WENC_TAP_C1) {
        const hipError_t e = hipMemcpy2DAsync(tap_dst, size_t(F) * d * 2, c1 + d, size_t(F + 2) * d * 2,
                                              size_t(F) * d * 2, nb, hipMemcpyDeviceToDevice, st);
        return e == hipSuccess ? WENC_OK : fail(&err, WENC_EHIP, "tap copy: %s", hipGetErrorString(e));
    }

    // conv2: output position t reads padded conv1 rows 2t .. 2t+2.
    g = wenc_gemm_args{};
    g.A = c1;
    g.a_batch_stride = int64_t(F + 2) * d;
    g.a_rows_per_batch = T;
    g.lda = 2 * d;
    g.W = W<uint16_t>(wl.conv2_w);
    g.ldw = 3 * d;
    g.bias = W<float>(wl.conv2_b);
    g.C = x;
    g.ldc = d;
    g.pos = W<float>(wl.pos);
    g.pos_rows = T;
    g.M = M;
    g.N = d;
    g.K = 3 * d;
    g.epilogue = WENC_EPI_CONV2;
    WENC_TRY(site(WENC_SITE_CONV2, st, [&] { return wk::launch_gemm(g, st, 0, cu_div); }));
    auto copy_x = [&](void *dst) {
        const hipError_t e = hipMemcpyAsync(dst, x, size_t(M) * d * 4, hipMemcpyDeviceToDevice, st);
        return e == hipSuccess ? WENC_OK : fail(&err, WENC_EHIP, "tap copy: %s", hipGetErrorString(e));
    };
    if (tap == WENC_TAP_STEM) return copy_x(tap_dst);

    const float q_scale = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
    for (int l = 0; l < c.n_layer; ++l) {
        const LayerOff &lo = wl.layers[l];
        WENC_TRY(site(WENC_SITE_LN1, st, [&] {
            return wk::launch_layernorm(x, W<float>(lo.ln1_g), W<float>(lo.ln1_b), xn, M, d, c.ln_eps, false, st);
        }));
        g = wenc_gemm_args{};
        g.A = xn;
        g.a_batch_stride = int64_t(T) * d;
        g.a_rows_per_batch = T;
        g.lda = d;
        g.W = W<uint16_t>(lo.wqkv);
        g.ldw = d;
        g.bias = W<float>(lo.bqkv);
        g.q = q;
        g.k = k;
        g.vt = vt;
        g.T = T;
        g.n_head = H;
        g.ldvt = ldvt;
        g.q_scale = q_scale;
        g.M = M;
        g.N = 3 * d;
        g.K = d;
        g.epilogue = WENC_EPI_QKV;
        WENC_TRY(site(WENC_SITE_QKV, st, [&] { return wk::launch_gemm(g, st, 0, cu_div); }));
        WENC_TRY(site(WENC_SITE_ATTN, st, [&] { return wk::launch_attention(q, k, vt, ao, nb, H, T, ldvt, st); }));
        g = wenc_gemm_args{};
        g.A = ao;
        g.a_batch_stride = int64_t(T) * d;
        g.a_rows_per_batch = T;
        g.lda = d;
        g.W = W<uint16_t>(lo.wo);
        g.ldw = d;
        g.bias = W<float>(lo.bo);
        g.C = x;
        g.ldc = d;
        g.M = M;
        g.N = d;
        g.K = d;
        g.epilogue = WENC_EPI_RESID;
        WENC_TRY(site(WENC_SITE_OPROJ, st, [&] { return wk::launch_gemm(g, st, 0, cu_div); }));
        WENC_TRY(site(WENC_SITE_LN2, st, [&] {
            return wk::launch_layernorm(x, W<float>(lo.ln2_g), W<float>(lo.ln2_b), xn, M, d, c.ln_eps, false, st);
        }));
        g = wenc_gemm_args{};
        g.A = xn;
        g.a_batch_stride = int64_t(T) * d;
        g.a_rows_per_batch = T;
        g.lda = d;
        g.W = W<uint16_t>(lo.fc1_w);
        g.ldw = d;
        g.bias = W<float>(lo.fc1_b);
        g.C = hb;
        g.c_batch_stride = int64_t(T) * Fd;
        g.c_rows_per_batch = T;
        g.ldc = Fd;
        g.M = M;
        g.N = Fd;
        g.K = d;
        g.epilogue = WENC_EPI_GELU_F16;
        WENC_TRY(site(WENC_SITE_FC1, st, [&] { return wk::launch_gemm(g, st, 1, cu_div); }));
        g = wenc_gemm_args{};
        g.A = hb;
        g.a_batch_stride = int64_t(T) * Fd;
        g.a_rows_per_batch = T;
        g.lda = Fd;
        g.W = W<uint16_t>(lo.fc2_w);
        g.ldw = Fd;
        g.bias = W<float>(lo.fc2_b);
        g.C = x;
        g.ldc = d;
        g.M = M;
        g.N = d;
        g.K = Fd;
        g.epilogue = WENC_EPI_RESID;
        WENC_TRY(site(WENC_SITE_FC2, st, [&] { return wk::launch_gemm(g, st, 1, cu_div); }));
        if (tap == WENC_TAP_BLOCK + l) return copy_x(tap_dst);
    }

    if (c.final_ln) {
        WENC_TRY(site(WENC_SITE_LNF, st, [&] {
            return wk::launch_layernorm(x, W<float>(wl.lnf_g), W<float>(wl.lnf_b), out, M, d, c.ln_eps, true, st);
        }));
        return WENC_OK;
    }
    return copy_x(out);
}

// Frees everything a handle owns (device memory, events, the stream) and
// the handle; the device must be idle for it.
static void release(wenc *h) {
    for (auto &r : h->prof_pending) {
        (void)hipEventDestroy(r.e0);
        (void)hipEventDestroy(r.e1);
    }
    for (auto e : h->event_pool) (void)hipEventDestroy(e);
    if (h->gexec) (void)hipGraphExecDestroy(h->gexec);
    if (h->cap) (void)hipStreamDestroy(h->cap);
    if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
    for (int i = 0; i + 1 < wenc::MAX_PARTS; ++i) {
        if (h->ev_join[i]) (void)hipEventDestroy(h->ev_join[i]);
        if (h->aux[i]) (void)hipStreamDestroy(h->aux[i]);
    }
    if (h->warena) (void)hipFree(h->warena);
    if (h->sarena) (void)hipFree(h->sarena);
    if (h->xarena) (void)hipFree(h->xarena);
    if (h->farena) (void)hipFree(h->farena);
    delete h;
}

extern "C" {

size_t wenc_weights_nbytes(const wenc_config *cfg) {
    if (config_error(cfg)) return 0;
    return 2 * blob_halves(*cfg);
}

int wenc_create(const wenc_config *cfg, wenc_t **out) {
    if (!out) return fail(nullptr, WENC_EINVAL, "wenc_create: out is NULL");
    *out = nullptr;
    if (const char *m = config_error(cfg)) return fail(nullptr, WENC_EINVAL, "wenc_create: %s", m);
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0)
        return fail(nullptr, WENC_ENODEV, "wenc_create: no HIP device (%s)", e != hipSuccess ? hipGetErrorString(e) : "count 0");
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(nullptr, WENC_ENODEV, "wenc_create: hipGetDevice: %s", hipGetErrorString(e));
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(nullptr, WENC_ENODEV, "wenc_create: hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(nullptr, WENC_ENODEV, "wenc_create: device %d is %s; this library is built for gfx950", dev,
                    prop.gcnArchName);

    wenc *h = new wenc();
    h->cfg = *cfg;
    h->device = dev;
    h->wl = weight_layout(*cfg);
    h->sl = scratch_layout(*cfg);
    const char *dbg = std::getenv("WENC_DEBUG_SYNC");
    h->debug_sync = dbg && dbg[0] == '1';
    // WENC_SPLIT_STREAMS=n splits a chunk's windows over n streams (1 keeps
    // every launch on the caller's stream; at most MAX_PARTS).
    if (const char *pp = std::getenv("WENC_SPLIT_STREAMS"))
        h->n_parts = std::max(1, std::min(std::atoi(pp), int(wenc::MAX_PARTS)));
    auto alloc = [&](char **p, size_t bytes, const char *what) -> int {
        const hipError_t ea = hipMalloc(reinterpret_cast<void **>(p), bytes);
        if (ea != hipSuccess) {
            (void)hipGetLastError();
            size_t fr = 0, tot = 0;
            (void)hipMemGetInfo(&fr, &tot);  // best effort: the message reports 0 if it fails
            *p = nullptr;
            return fail(nullptr, WENC_ENOMEM, "wenc_create: cannot allocate %zu bytes of %s (device has %zu free of %zu)",
                        bytes, what, fr, tot);
        }
        return WENC_OK;
    };
    int rc = WENC_OK;
    e = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking);
    for (int i = 0; i + 1 < h->n_parts && e == hipSuccess; ++i) {
        e = hipStreamCreateWithFlags(&h->aux[i], hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_join[i], hipEventDisableTiming);
    }
    if (e != hipSuccess) rc = fail(nullptr, WENC_EHIP, "wenc_create: stream or event: %s", hipGetErrorString(e));
    if (rc == WENC_OK) rc = alloc(&h->warena, h->wl.total, "weights");
    if (rc == WENC_OK) rc = alloc(&h->sarena, h->sl.total, "activation scratch");
    if (rc == WENC_OK) {
        // WENC_POISON_SCRATCH=1 fills the activations with all-ones bytes (NaN
        // in fp16 and fp32) so that a read of never-written scratch shows up.
        const char *poison = std::getenv("WENC_POISON_SCRATCH");
        e = hipMemset(h->sarena, poison && poison[0] == '1' ? 0xff : 0, h->sl.total);
        if (e != hipSuccess) rc = fail(nullptr, WENC_EHIP, "wenc_create: hipMemset: %s", hipGetErrorString(e));
    }
    if (rc == WENC_OK && !wk::logmel_check(1, cfg->n_frames, cfg->n_mels)) {
        const FrontendTables t = frontend_tables(cfg->n_mels);
        Bump fb;
        const size_t tab = fb.take(4 * t.tab.size());
        h->f_win = fb.take(4 * t.win.size());
        h->f_mwt = fb.take(4 * t.mwt.size());
        h->f_mstart = fb.take(4 * t.mstart.size());
        h->f_nch = t.nch;
        h->f_blk = fb.take(4 * size_t(cfg->max_batch) * wk::logmel_tiles(cfg->n_frames));
        // every filter's window lies within the 201 bins (otherwise the handle
        // has no frontend and wenc_log_mel reports it)
        bool ok = 16 * t.nch <= 201 && cfg->n_mels * (t.nch - 1) * 16 <= wk::LOGMEL_MAX_EXTRA;
        for (int i = 0; ok && i < cfg->n_mels; ++i) ok = t.mstart[i] >= 0 && t.mstart[i] + 16 * t.nch <= 201;
        if (ok) rc = alloc(&h->farena, fb.off, "log-mel tables");
        if (ok && rc == WENC_OK) {
            e = hipMemcpy(h->farena + tab, t.tab.data(), 4 * t.tab.size(), hipMemcpyHostToDevice);
            if (e == hipSuccess) e = hipMemcpy(h->farena + h->f_win, t.win.data(), 4 * t.win.size(), hipMemcpyHostToDevice);
            if (e == hipSuccess) e = hipMemcpy(h->farena + h->f_mwt, t.mwt.data(), 4 * t.mwt.size(), hipMemcpyHostToDevice);
            if (e == hipSuccess)
                e = hipMemcpy(h->farena + h->f_mstart, t.mstart.data(), 4 * t.mstart.size(), hipMemcpyHostToDevice);
            if (e != hipSuccess) rc = fail(nullptr, WENC_EHIP, "wenc_create: table upload: %s", hipGetErrorString(e));
        }
    }
    if (rc != WENC_OK) {
        release(h);
        return rc;
    }
    *out = h;
    return WENC_OK;
}

int wenc_load(wenc_t *h, const void *blob, size_t nbytes) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_load: handle is NULL");
    if (!blob) return fail(&h->err, WENC_EINVAL, "wenc_load: blob is NULL");
    const wenc_config &c = h->cfg;
    const size_t want = 2 * blob_halves(c);
    if (nbytes != want)
        return fail(&h->err, WENC_EINVAL, "wenc_load: blob has %zu bytes, this config needs exactly %zu", nbytes, want);
    const size_t d = c.d_model, F = c.d_ff, nm = c.n_mels, T = c.n_ctx;
    std::vector<char> host(h->wl.total, 0);
    const uint16_t *src = static_cast<const uint16_t *>(blob);
    auto f32 = [&](size_t off, size_t n) {
        float *dst = reinterpret_cast<float *>(host.data() + off);
        for (size_t i = 0; i < n; ++i) dst[i] = half_to_float(src[i]);
        src += n;
    };
    auto f16 = [&](size_t off, size_t n) {
        std::memcpy(host.data() + off, src, 2 * n);
        src += n;
    };
    // conv taps [out][in][k] -> [out][k][in] so a GEMM row reads k-major windows.
    auto conv = [&](size_t off, size_t cout, size_t cin) {
        uint16_t *dst = reinterpret_cast<uint16_t *>(host.data() + off);
        for (size_t o = 0; o < cout; ++o)
            for (size_t ci = 0; ci < cin; ++ci)
                for (size_t j = 0; j < 3; ++j) dst[o * 3 * cin + j * cin + ci] = src[(o * cin + ci) * 3 + j];
        src += cout * cin * 3;
    };
    conv(h->wl.conv1_w, d, nm);
    f32(h->wl.conv1_b, d);
    conv(h->wl.conv2_w, d, d);
    f32(h->wl.conv2_b, d);
    f32(h->wl.pos, T * d);
    for (int l = 0; l < c.n_layer; ++l) {
        const LayerOff &lo = h->wl.layers[l];
        f32(lo.ln1_g, d);
        f32(lo.ln1_b, d);
        f16(lo.wqkv, d * d);                 // wq -> rows [0, d)
        f32(lo.bqkv, d);                     // bq
        f16(lo.wqkv + 2 * d * d, d * d);     // wk -> rows [d, 2d); k_proj has no bias (left 0)
        f16(lo.wqkv + 4 * d * d, d * d);     // wv -> rows [2d, 3d)
        f32(lo.bqkv + 4 * 2 * d, d);         // bv
        f16(lo.wo, d * d);
        f32(lo.bo, d);
        f32(lo.ln2_g, d);
        f32(lo.ln2_b, d);
        f16(lo.fc1_w, F * d);
        f32(lo.fc1_b, F);
        f16(lo.fc2_w, d * F);
        f32(lo.fc2_b, d);
    }
    f32(h->wl.lnf_g, d);
    f32(h->wl.lnf_b, d);
    hipError_t e = hipSetDevice(h->device);
    if (e != hipSuccess) return fail(&h->err, WENC_EHIP, "wenc_load: hipSetDevice: %s", hipGetErrorString(e));
    if (h->loaded) {
        // A forward may still be queued on any stream (torch's side streams do
        // not wait for the null stream's copy): let it finish on the old weights.
        e = hipDeviceSynchronize();
        if (e != hipSuccess)
            return fail(&h->err, WENC_EHIP, "wenc_load: waiting for enqueued work: %s", hipGetErrorString(e));
    }
    // From here the arena holds neither the old nor (until the copy ends) the
    // new weights: a failed upload leaves the handle unloaded.
    h->loaded = false;
    e = hipMemcpy(h->warena, host.data(), host.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(&h->err, WENC_EHIP, "wenc_load: upload failed: %s", hipGetErrorString(e));
    h->loaded = true;
    return WENC_OK;
}

// Every chunk of a checked forward, in order, on stream st.
static int enqueue_forward(wenc_t *h, const float *mel, int32_t batch, int32_t n_ctx, float *out, hipStream_t st) {
    const wenc_config &c = h->cfg;
    const int cap = h->chunk_cap(n_ctx);
    for (int b0 = 0; b0 < batch; b0 += cap) {
        const int nb = batch - b0 < cap ? batch - b0 : cap;
        WENC_TRY(h->forward_chunk(mel + size_t(b0) * 2 * n_ctx * c.n_mels, nb, n_ctx,
                                  out + size_t(b0) * n_ctx * c.d_model, st, -1, nullptr));
    }
    return WENC_OK;
}

static int forward_impl(wenc_t *h, const float *mel, int32_t batch, int32_t n_ctx, float *out, void *stream, int tap,
                        void *tap_dst) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_forward: handle is NULL");
    if (!h->loaded) return fail(&h->err, WENC_ESTATE, "wenc_forward: no weights loaded (call wenc_load first)");
    if (batch < 0) return fail(&h->err, WENC_EINVAL, "wenc_forward: batch %d < 0", batch);
    const wenc_config &c = h->cfg;
    if (n_ctx < 1 || n_ctx > c.n_ctx)
        return fail(&h->err, WENC_EINVAL, "wenc_forward_ctx: n_ctx %d outside [1, %d]", n_ctx, c.n_ctx);
    if (batch == 0) return WENC_OK;
    if (!mel) return fail(&h->err, WENC_EINVAL, "wenc_forward: mel is NULL");
    if (misaligned(mel, 16)) return fail(&h->err, WENC_EINVAL, "wenc_forward: mel must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (tap >= 0) {
        if (!tap_dst) return fail(&h->err, WENC_EINVAL, "wenc_forward_tap: dst is NULL");
        if (tap > WENC_TAP_BLOCK + c.n_layer - 1)
            return fail(&h->err, WENC_EINVAL, "wenc_forward_tap: tap %d out of range", tap);
        if (batch > c.max_batch)
            return fail(&h->err, WENC_EINVAL, "wenc_forward_tap: batch %d > max_batch %d", batch, c.max_batch);
        return h->forward_chunk(mel, batch, n_ctx, nullptr, st, tap, tap_dst);
    }
    if (!out) return fail(&h->err, WENC_EINVAL, "wenc_forward: out is NULL");
    if (misaligned(out, 16)) return fail(&h->err, WENC_EINVAL, "wenc_forward: out must be 16-byte aligned");
    return enqueue_forward(h, mel, batch, n_ctx, out, st);
}

int wenc_forward(wenc_t *h, const float *mel, int32_t batch, float *out, void *stream) {
    return forward_impl(h, mel, batch, h ? h->cfg.n_ctx : 1, out, stream, -1, nullptr);
}

int wenc_forward_ctx(wenc_t *h, const float *mel, int32_t batch, int32_t n_ctx, float *out, void *stream) {
    return forward_impl(h, mel, batch, n_ctx, out, stream, -1, nullptr);
}

int wenc_forward_graph(wenc_t *h, const float *mel, int32_t batch, int32_t n_ctx, float *out, void *stream) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_forward_graph: handle is NULL");
    if (!h->loaded) return fail(&h->err, WENC_ESTATE, "wenc_forward_graph: no weights loaded (call wenc_load first)");
    const wenc_config &c = h->cfg;
    if (batch < 0) return fail(&h->err, WENC_EINVAL, "wenc_forward_graph: batch %d < 0", batch);
    if (n_ctx < 1 || n_ctx > c.n_ctx)
        return fail(&h->err, WENC_EINVAL, "wenc_forward_graph: n_ctx %d outside [1, %d]", n_ctx, c.n_ctx);
    if (batch == 0) return WENC_OK;
    if (!mel || !out) return fail(&h->err, WENC_EINVAL, "wenc_forward_graph: mel and out must be non-null");
    if (misaligned(mel, 16) || misaligned(out, 16))
        return fail(&h->err, WENC_EINVAL, "wenc_forward_graph: mel and out must be 16-byte aligned");
    if (h->prof_mask || h->debug_sync)
        return fail(&h->err, WENC_ESTATE,
                    "wenc_forward_graph: not while per-launch profiling or WENC_DEBUG_SYNC is on (neither can be "
                    "recorded into a graph)");
    hipError_t e = hipSetDevice(h->device);
    if (e != hipSuccess) return fail(&h->err, WENC_EHIP, "wenc_forward_graph: hipSetDevice: %s", hipGetErrorString(e));
    if (!h->gexec || h->g_mel != mel || h->g_out != out || h->g_batch != batch || h->g_nctx != n_ctx) {
        // record the forward once for these buffers and sizes
        if (h->gexec) {
            e = hipGraphExecDestroy(h->gexec);
            h->gexec = nullptr;
            if (e != hipSuccess)
                return fail(&h->err, WENC_EHIP, "wenc_forward_graph: releasing the previous graph: %s", hipGetErrorString(e));
        }
        e = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) return fail(&h->err, WENC_EHIP, "wenc_forward_graph: begin capture: %s", hipGetErrorString(e));
        const int rc = enqueue_forward(h, mel, batch, n_ctx, out, h->cap);
        hipGraph_t g = nullptr;
        e = hipStreamEndCapture(h->cap, &g);
        if (rc != WENC_OK || e != hipSuccess || !g) {
            if (g) (void)hipGraphDestroy(g);
            if (rc != WENC_OK) return rc;
            return fail(&h->err, WENC_EHIP, "wenc_forward_graph: end capture: %s", hipGetErrorString(e));
        }
        e = hipGraphInstantiate(&h->gexec, g, nullptr, nullptr, 0);
        (void)hipGraphDestroy(g);  // the executable graph keeps what it needs
        if (e != hipSuccess) {
            h->gexec = nullptr;
            return fail(&h->err, WENC_EHIP, "wenc_forward_graph: instantiate: %s", hipGetErrorString(e));
        }
        h->g_mel = mel;
        h->g_out = out;
        h->g_batch = batch;
        h->g_nctx = n_ctx;
    }
    e = hipGraphLaunch(h->gexec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(&h->err, WENC_EHIP, "wenc_forward_graph: launch: %s", hipGetErrorString(e));
    return WENC_OK;
}

int wenc_forward_tap(wenc_t *h, const float *mel, int32_t batch, int32_t tap, void *dst, void *stream) {
    if (h && tap < 0) return fail(&h->err, WENC_EINVAL, "wenc_forward_tap: tap %d < 0", tap);
    return forward_impl(h, mel, batch, h ? h->cfg.n_ctx : 1, nullptr, stream, tap, dst);
}

size_t wenc_cross_nbytes(const wenc_config *cfg, int32_t n_dec_layer) {
    if (config_error(cfg) || n_dec_layer <= 0 || n_dec_layer > 4096) return 0;
    const size_t d = cfg->d_model;
    return 2 * size_t(n_dec_layer) * (2 * d * d + d);
}

int wenc_load_cross(wenc_t *h, int32_t n_dec_layer, const void *blob, size_t nbytes) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_load_cross: handle is NULL");
    if (!blob) return fail(&h->err, WENC_EINVAL, "wenc_load_cross: blob is NULL");
    const size_t want = wenc_cross_nbytes(&h->cfg, n_dec_layer);
    if (want == 0) return fail(&h->err, WENC_EINVAL, "wenc_load_cross: n_dec_layer %d outside [1, 4096]", n_dec_layer);
    if (nbytes != want)
        return fail(&h->err, WENC_EINVAL, "wenc_load_cross: blob is %zu bytes, expected exactly %zu", nbytes, want);
    const size_t d = h->cfg.d_model;
    const size_t stride = (4 * d * d + 8 * d + 255) & ~size_t(255);
    std::vector<char> host(stride * n_dec_layer, 0);
    const uint16_t *src = static_cast<const uint16_t *>(blob);
    for (int l = 0; l < n_dec_layer; ++l) {
        char *dst = host.data() + l * stride;
        std::memcpy(dst, src, 2 * d * d * 2);  // x_wk then x_wv: rows [0, d) and [d, 2d) of W_kv
        src += 2 * d * d;
        float *bias = reinterpret_cast<float *>(dst + 4 * d * d);  // [0; x_bv]: x_wk has no bias
        for (size_t i = 0; i < d; ++i) bias[d + i] = half_to_float(src[i]);
        src += d;
    }
    hipError_t e = hipSetDevice(h->device);
    if (e != hipSuccess) return fail(&h->err, WENC_EHIP, "wenc_load_cross: hipSetDevice: %s", hipGetErrorString(e));
    if (h->xarena) {
        e = hipDeviceSynchronize();  // no enqueued work may still read the old weights
        if (e == hipSuccess) e = hipFree(h->xarena);
        if (e != hipSuccess)
            return fail(&h->err, WENC_EHIP, "wenc_load_cross: releasing the previous weights: %s", hipGetErrorString(e));
        h->xarena = nullptr;
        h->n_dec = 0;
    }
    e = hipMalloc(reinterpret_cast<void **>(&h->xarena), host.size());
    if (e != hipSuccess) {
        (void)hipGetLastError();
        size_t fr = 0, tot = 0;
        (void)hipMemGetInfo(&fr, &tot);  // best effort: the message reports 0 if it fails
        h->xarena = nullptr;
        return fail(&h->err, WENC_ENOMEM, "wenc_load_cross: cannot allocate %zu bytes (device has %zu free of %zu)",
                    host.size(), fr, tot);
    }
    e = hipMemcpy(h->xarena, host.data(), host.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(&h->err, WENC_EHIP, "wenc_load_cross: upload failed: %s", hipGetErrorString(e));
    h->n_dec = n_dec_layer;
    h->x_stride = stride;
    return WENC_OK;
}

int wenc_prepare_cross(wenc_t *h, const float *memory, int32_t batch, int32_t n_ctx, void *xk, void *xv,
                       void *stream) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_prepare_cross: handle is NULL");
    if (!h->xarena) return fail(&h->err, WENC_ESTATE, "wenc_prepare_cross: no cross weights (call wenc_load_cross first)");
    const wenc_config &c = h->cfg;
    if (batch < 0) return fail(&h->err, WENC_EINVAL, "wenc_prepare_cross: batch %d < 0", batch);
    if (n_ctx < 1 || n_ctx > c.n_ctx)
        return fail(&h->err, WENC_EINVAL, "wenc_prepare_cross: n_ctx %d outside [1, %d]", n_ctx, c.n_ctx);
    if (batch == 0) return WENC_OK;
    if (!memory || !xk || !xv) return fail(&h->err, WENC_EINVAL, "wenc_prepare_cross: memory, xk and xv must be non-null");
    if (misaligned(memory, 16) || misaligned(xk, 16) || misaligned(xv, 16))
        return fail(&h->err, WENC_EINVAL, "wenc_prepare_cross: memory, xk and xv must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int d = c.d_model, T = n_ctx;
    const int cap = h->chunk_cap(T);
    uint16_t *mh = h->S<uint16_t>(h->sl.xn);  // the memory in fp16, [nb * T][d]
    for (int b0 = 0; b0 < batch; b0 += cap) {
        const int nb = batch - b0 < cap ? batch - b0 : cap;
        const int64_t rows = int64_t(nb) * T;
        WENC_TRY(h->site(WENC_SITE_XCVT, st, [&] {
            return wk::launch_to_f16(memory + size_t(b0) * T * d, mh, rows * d, st);
        }));
        for (int l = 0; l < h->n_dec; ++l) {
            const char *lw = h->xarena + l * h->x_stride;
            const size_t off = (size_t(l) * batch + b0) * size_t(T) * d;
            wenc_gemm_args g{};
            g.A = mh;
            g.a_batch_stride = int64_t(T) * d;
            g.a_rows_per_batch = T;
            g.lda = d;
            g.W = reinterpret_cast<const uint16_t *>(lw);
            g.ldw = d;
            g.bias = reinterpret_cast<const float *>(lw + size_t(4) * d * d);
            g.C = static_cast<uint16_t *>(xk) + off;
            g.C2 = static_cast<uint16_t *>(xv) + off;
            g.n_split = d;
            g.ldc = d;
            g.M = int(rows);
            g.N = 2 * d;
            g.K = d;
            g.epilogue = WENC_EPI_KV;
            WENC_TRY(h->site(WENC_SITE_XKV, st, [&] { return wk::launch_gemm(g, st); }));
        }
    }
    return WENC_OK;
}

int wenc_cross_attend(wenc_t *h, const void *q, const void *xk, const void *xv, int32_t batch, int32_t n_q,
                      int32_t n_ctx, void *out, void *stream) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_cross_attend: handle is NULL");
    const wenc_config &c = h->cfg;
    if (const char *m = wk::xattn_check(batch, c.n_head, n_q, n_ctx))
        return fail(&h->err, WENC_EINVAL, "wenc_cross_attend: %s", m);
    if (n_ctx > c.n_ctx) return fail(&h->err, WENC_EINVAL, "wenc_cross_attend: n_ctx %d > %d", n_ctx, c.n_ctx);
    if (batch == 0) return WENC_OK;
    if (!q || !xk || !xv || !out) return fail(&h->err, WENC_EINVAL, "wenc_cross_attend: null pointer");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(xk) | reinterpret_cast<uintptr_t>(xv) |
         reinterpret_cast<uintptr_t>(out)) & 15)
        return fail(&h->err, WENC_EINVAL, "wenc_cross_attend: q, xk, xv and out must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int d = c.d_model;
    // the partials live in the fp16 LayerNorm-output region of the scratch
    const size_t room = size_t(2) * c.max_batch * c.n_ctx * d;
    const size_t per = wk::xattn_part_bytes(1, c.n_head, n_q, n_ctx);
    if (per > room) return fail(&h->err, WENC_EINVAL, "wenc_cross_attend: the scratch cannot hold one item's partials");
    const int cap = int(std::max<size_t>(1, std::min<size_t>(room / per, size_t(batch))));
    float *part = h->S<float>(h->sl.xn);
    for (int b0 = 0; b0 < batch; b0 += cap) {
        const int nb = batch - b0 < cap ? batch - b0 : cap;
        const size_t qo = size_t(b0) * n_q * d, ko = size_t(b0) * n_ctx * d;
        WENC_TRY(h->site(WENC_SITE_XATT, st, [&] {
            return wk::launch_xattn(static_cast<const uint16_t *>(q) + qo, static_cast<const uint16_t *>(xk) + ko,
                                    static_cast<const uint16_t *>(xv) + ko, static_cast<uint16_t *>(out) + qo, part, nb,
                                    c.n_head, n_q, n_ctx, st);
        }));
    }
    return WENC_OK;
}

int wenc_argmax(wenc_t *h, const float *logits, int32_t rows, int32_t n_vocab, int64_t ld, int32_t *out,
                void *stream) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_argmax: handle is NULL");
    const wenc_config &c = h->cfg;
    if (const char *m = wk::argmax_check(rows, n_vocab, ld)) return fail(&h->err, WENC_EINVAL, "wenc_argmax: %s", m);
    if (rows == 0) return WENC_OK;
    if (!logits || !out) return fail(&h->err, WENC_EINVAL, "wenc_argmax: null pointer");
    if ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(out)) & 3)
        return fail(&h->err, WENC_EINVAL, "wenc_argmax: logits and out must be 4-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the chunk keys live in the fp16 LayerNorm-output region of the scratch
    const size_t room = size_t(2) * c.max_batch * c.n_ctx * c.d_model;
    const size_t per = size_t(wk::argmax_chunks(n_vocab)) * sizeof(uint64_t);
    if (per > room) return fail(&h->err, WENC_EINVAL, "wenc_argmax: the scratch cannot hold one row's chunk keys");
    const int cap = int(std::max<size_t>(1, std::min<size_t>(room / per, size_t(rows))));
    uint64_t *part = h->S<uint64_t>(h->sl.xn);
    for (int r0 = 0; r0 < rows; r0 += cap) {
        const int nr = rows - r0 < cap ? rows - r0 : cap;
        WENC_TRY(h->site(WENC_SITE_ARGMAX, st, [&] {
            return wk::launch_argmax(logits + size_t(r0) * size_t(ld), nr, n_vocab, ld, part, out + r0, st);
        }));
    }
    return WENC_OK;
}

int wenc_log_mel(wenc_t *h, const float *audio, int32_t batch, float *mel, void *stream) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_log_mel: handle is NULL");
    const wenc_config &c = h->cfg;
    if (const char *m = wk::logmel_check(batch, c.n_frames, c.n_mels))
        return fail(&h->err, WENC_EINVAL, "wenc_log_mel: %s", m);
    if (!h->farena) return fail(&h->err, WENC_ESTATE, "wenc_log_mel: frontend tables missing");
    if (batch == 0) return WENC_OK;
    if (!audio || !mel) return fail(&h->err, WENC_EINVAL, "wenc_log_mel: audio and mel must be non-null");
    if (misaligned(audio, 4) || misaligned(mel, 16))
        return fail(&h->err, WENC_EINVAL, "wenc_log_mel: audio must be 4-byte and mel 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const float *tab = reinterpret_cast<const float *>(h->farena);
    const float *win = reinterpret_cast<const float *>(h->farena + h->f_win);
    const float *mwt = reinterpret_cast<const float *>(h->farena + h->f_mwt);
    const int *mstart = reinterpret_cast<const int *>(h->farena + h->f_mstart);
    float *blk = reinterpret_cast<float *>(h->farena + h->f_blk);
    for (int b0 = 0; b0 < batch; b0 += c.max_batch) {
        const int nb = batch - b0 < c.max_batch ? batch - b0 : c.max_batch;
        WENC_TRY(h->site(WENC_SITE_MEL, st, [&] {
            return wk::launch_logmel(audio + size_t(b0) * c.n_frames * 160, nb, c.n_frames, tab, win, mwt, mstart,
                                     h->f_nch, c.n_mels, mel + size_t(b0) * c.n_frames * c.n_mels, blk, st);
        }));
    }
    return WENC_OK;
}

void wenc_destroy(wenc_t *h) {
    if (!h) return;
    // teardown: errors cannot be acted on here, every release is attempted
    (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();
    release(h);
}

const char *wenc_last_error(const wenc_t *h) {
    if (h) return h->err.c_str();
    return g_err;
}

int wenc_argmax_noalloc(const float *logits, int32_t rows, int32_t n_vocab, int64_t ld, int32_t *out, void *stream) {
    if (const char *m = wk::argmax_check(rows, n_vocab, ld)) return fail(nullptr, WENC_EINVAL, "wenc_argmax_noalloc: %s", m);
    const int64_t nc = wk::argmax_chunks(n_vocab);
    if (nc > 1 && nc > wk::ARGMAX_STATIC_KEYS)
        return fail(nullptr, WENC_EINVAL,
                    "wenc_argmax_noalloc: n_vocab %d needs %lld chunk keys per row, beyond the static scratch of %lld "
                    "(n_vocab <= %lld)",
                    n_vocab, (long long)nc, (long long)wk::ARGMAX_STATIC_KEYS, (long long)wk::ARGMAX_STATIC_KEYS * 2048);
    if (rows == 0) return WENC_OK;
    if (!logits || !out) return fail(nullptr, WENC_EINVAL, "wenc_argmax_noalloc: null pointer");
    if (misaligned(logits, 4) || misaligned(out, 4))
        return fail(nullptr, WENC_EINVAL, "wenc_argmax_noalloc: logits and out must be 4-byte aligned");
    uint64_t *part = nullptr;
    hipError_t e = wk::static_scratch(&part);
    if (e != hipSuccess) return fail(nullptr, WENC_EHIP, "wenc_argmax_noalloc: scratch address: %s", hipGetErrorString(e));
    hipStream_t st = static_cast<hipStream_t>(stream);
    // rows in passes of what the scratch holds (each pass's keys are all
    // written by its first kernel before its second reads them)
    const int64_t cap = nc > 1 ? std::min<int64_t>(wk::ARGMAX_STATIC_KEYS / nc, rows) : rows;
    for (int64_t r0 = 0; r0 < rows; r0 += cap) {
        const int nr = int(std::min<int64_t>(cap, rows - r0));
        e = wk::launch_argmax(logits + r0 * ld, nr, n_vocab, ld, part, out + r0, st);
        if (e != hipSuccess) return fail(nullptr, WENC_EHIP, "wenc_argmax_noalloc: launch: %s", hipGetErrorString(e));
    }
    return WENC_OK;
}

int wenc_k_layernorm(const float *x, const float *gamma, const float *beta, void *y, int32_t rows, int32_t d, float eps,
                     int32_t out_f32, void *stream) {
    if (const char *m = wk::layernorm_check(rows, d)) return fail(nullptr, WENC_EINVAL, "%s", m);
    if (rows > 0 && (!x || !gamma || !beta || !y)) return fail(nullptr, WENC_EINVAL, "layernorm: null pointer");
    const hipError_t e = wk::launch_layernorm(x, gamma, beta, y, rows, d, eps, out_f32 != 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? WENC_OK : fail(nullptr, WENC_EHIP, "layernorm: %s", hipGetErrorString(e));
}

int wenc_k_gemm(const wenc_gemm_args *args, void *stream) {
    if (!args) return fail(nullptr, WENC_EINVAL, "gemm: args is NULL");
    if (const char *m = wk::gemm_check(*args)) return fail(nullptr, WENC_EINVAL, "%s", m);
    const hipError_t e = wk::launch_gemm(*args, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? WENC_OK : fail(nullptr, WENC_EHIP, "gemm: %s", hipGetErrorString(e));
}

int wenc_k_gemm_mode(int32_t tile, int32_t split) {
    if (wk::gemm_mode(tile, split) != 0) return fail(nullptr, WENC_EINVAL, "gemm mode: tile must be -1, 0, 1 or 2 and split 0 or 1");
    return WENC_OK;
}

int wenc_k_gemm_plan(int32_t M, int32_t N, int32_t cus, int32_t tile, int32_t split, int32_t streams,
                     int32_t *big_rows) {
    if (M < 1 || N < 1 || cus < 1 || tile < -1 || tile > 1 || split < 0 || split > 1 || streams < 1 || !big_rows)
        return fail(nullptr, WENC_EINVAL,
                    "gemm plan: need M, N, cus, streams >= 1, tile in [-1, 1], split in [0, 1], big_rows");
    const wk::GemmPlan p = wk::gemm_plan(M, N, cus, tile, split, streams);
    *big_rows = p.big_rows;
    return p.kind;
}

int wenc_k_logmel_tables(int32_t n_mels, int32_t *nch, int32_t *mstart, float *mwt, int64_t mwt_cap) {
    if (const char *m = wk::logmel_check(1, 2, n_mels)) return fail(nullptr, WENC_EINVAL, "logmel tables: %s", m);
    if (!nch) return fail(nullptr, WENC_EINVAL, "logmel tables: nch is NULL");
    const FrontendTables t = frontend_tables(n_mels);
    *nch = t.nch;
    if (!mstart || !mwt) return WENC_OK;
    if (mwt_cap < int64_t(t.mwt.size()))
        return fail(nullptr, WENC_EINVAL, "logmel tables: mwt holds %lld floats, %zu needed", (long long)mwt_cap,
                    t.mwt.size());
    std::copy(t.mstart.begin(), t.mstart.end(), mstart);
    std::copy(t.mwt.begin(), t.mwt.end(), mwt);
    return WENC_OK;
}

int wenc_k_attention(const uint16_t *q, const uint16_t *k, const uint16_t *vt, uint16_t *ao, int32_t batch,
                     int32_t n_head, int32_t T, int32_t ldvt, void *stream) {
    if (const char *m = wk::attention_check(batch, n_head, T, ldvt)) return fail(nullptr, WENC_EINVAL, "%s", m);
    if (batch > 0 && (!q || !k || !vt || !ao)) return fail(nullptr, WENC_EINVAL, "attention: null pointer");
    const hipError_t e = wk::launch_attention(q, k, vt, ao, batch, n_head, T, ldvt, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? WENC_OK : fail(nullptr, WENC_EHIP, "attention: %s", hipGetErrorString(e));
}

int wenc_profile(wenc_t *h, uint32_t site_mask) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_profile: handle is NULL");
    h->prof_mask = site_mask & ((1u << WENC_N_SITES) - 1);
    return WENC_OK;
}

int wenc_profile_read(wenc_t *h, double *ms_total, int64_t *launches) {
    if (!h) return fail(nullptr, WENC_EINVAL, "wenc_profile_read: handle is NULL");
    if (!ms_total || !launches) return fail(&h->err, WENC_EINVAL, "wenc_profile_read: null output array");
    for (int s = 0; s < WENC_N_SITES; ++s) {
        ms_total[s] = 0.0;
        launches[s] = 0;
    }
    int rc = WENC_OK;
    // Each launch as an interval [start, end] in ms after the first recorded
    // event; a site's time is the length of the union of its intervals, so
    // launches of one site that overlap on different streams count once.
    std::vector<std::vector<std::pair<float, float>>> iv(WENC_N_SITES);
    const hipEvent_t ref = h->prof_pending.empty() ? nullptr : h->prof_pending.front().e0;
    for (auto &r : h->prof_pending) {
        float t0 = 0.f, t1 = 0.f;
        hipError_t e = hipEventSynchronize(r.e1);
        if (e == hipSuccess) e = hipEventElapsedTime(&t0, ref, r.e0);
        if (e == hipSuccess) e = hipEventElapsedTime(&t1, ref, r.e1);
        if (e != hipSuccess && rc == WENC_OK) rc = fail(&h->err, WENC_EHIP, "wenc_profile_read: %s", hipGetErrorString(e));
        if (e == hipSuccess) iv[r.site].push_back({t0, std::max(t0, t1)});
        launches[r.site] += 1;
        h->event_pool.push_back(r.e0);
        h->event_pool.push_back(r.e1);
    }
    h->prof_pending.clear();
    for (int s = 0; s < WENC_N_SITES; ++s) {
        std::sort(iv[s].begin(), iv[s].end());
        double total = 0.0, lo = 0.0, hi = -1.0;
        for (const auto &x : iv[s]) {
            if (x.first > hi) {
                if (hi >= lo) total += hi - lo;
                lo = x.first;
                hi = x.second;
            } else {
                hi = std::max<double>(hi, x.second);
            }
        }
        if (hi >= lo) total += hi - lo;
        ms_total[s] = total;
    }
    return rc;
}

}  // extern "C"
