// Host-side checks of libwenc's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (the device code is not built).
// Every call here runs host logic only -- configuration and argument
// validation, blob sizes, the GEMM tile planner, the log-mel filter tables,
// error messages -- and must return the documented status without a GPU
// (wenc_create on a valid configuration reports the missing device).
// Exit status 0 and no sanitizer report mean the host logic is clean.
#include "wenc.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

namespace {

int failures = 0;

#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);   \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

wenc_config shape(int n_mels, int d, int layers, int max_batch = 4) {
    wenc_config c{};
    c.n_mels = n_mels;
    c.d_model = d;
    c.n_head = d / 64;
    c.head_dim = 64;
    c.d_ff = 4 * d;
    c.n_layer = layers;
    c.n_frames = 3000;
    c.n_ctx = 1500;
    c.ln_eps = 1e-5f;
    c.final_ln = 1;
    c.max_batch = max_batch;
    return c;
}

// The blob layout wenc.h documents, counted field by field (fp16 halves).
size_t documented_bytes(const wenc_config &c) {
    const size_t d = c.d_model, F = c.d_ff, nm = c.n_mels, T = c.n_ctx;
    size_t h = d * nm * 3 + d + d * d * 3 + d + T * d;
    for (int l = 0; l < c.n_layer; ++l)
        h += d + d + d * d + d + d * d + d * d + d + d * d + d + d + d + F * d + F + d * F + d;
    h += 2 * d;
    return 2 * h;
}

bool has_message() { return std::strlen(wenc_last_error(nullptr)) > 0; }

void sizes_and_configs() {
    // the Whisper family: tiny, base, small, medium, large-v3
    const wenc_config fam[] = {shape(80, 384, 4), shape(80, 512, 6), shape(80, 768, 12), shape(80, 1024, 24),
                               shape(128, 1280, 32)};
    for (const wenc_config &c : fam) {
        CHECK(wenc_weights_nbytes(&c) == documented_bytes(c));
        CHECK(wenc_cross_nbytes(&c, 4) == size_t(4) * 2 * (2 * size_t(c.d_model) * c.d_model + c.d_model));
        CHECK(wenc_cross_nbytes(&c, 0) == 0 && wenc_cross_nbytes(&c, -1) == 0);
    }
    CHECK(wenc_weights_nbytes(nullptr) == 0);

    // each invalid field on its own: size 0, wenc_create EINVAL with a message
    std::vector<wenc_config> bad;
    auto vary = [&](auto edit) {
        wenc_config c = shape(80, 384, 4);
        edit(c);
        bad.push_back(c);
    };
    vary([](wenc_config &c) { c.head_dim = 32; });
    vary([](wenc_config &c) { c.d_model = 400; });
    vary([](wenc_config &c) { c.n_head = 0; });
    vary([](wenc_config &c) { c.n_mels = 7; });
    vary([](wenc_config &c) { c.n_mels = 0; });
    vary([](wenc_config &c) { c.d_ff = 12; });
    vary([](wenc_config &c) { c.n_layer = -1; });
    vary([](wenc_config &c) { c.n_frames = 3001; });
    vary([](wenc_config &c) { c.n_ctx = 0; c.n_frames = 0; });
    vary([](wenc_config &c) { c.ln_eps = 0.f; });
    vary([](wenc_config &c) { c.ln_eps = std::nanf(""); });
    vary([](wenc_config &c) { c.final_ln = 2; });
    vary([](wenc_config &c) { c.max_batch = 0; });
    vary([](wenc_config &c) { c.max_batch = 6000; });
    vary([](wenc_config &c) { c.d_model = 64 * 40; c.n_head = 40; });
    for (const wenc_config &c : bad) {
        CHECK(wenc_weights_nbytes(&c) == 0);
        wenc_t *h = reinterpret_cast<wenc_t *>(uintptr_t(1));
        CHECK(wenc_create(&c, &h) == WENC_EINVAL && h == nullptr && has_message());
    }
    CHECK(wenc_create(nullptr, nullptr) == WENC_EINVAL);

    // a valid shape reaches the device check: no device here, or a real one
    wenc_config ok = shape(80, 384, 4, 2);
    wenc_t *h = nullptr;
    const int rc = wenc_create(&ok, &h);
    CHECK(rc == WENC_ENODEV || rc == WENC_OK || rc == WENC_ENOMEM);
    if (rc == WENC_OK) wenc_destroy(h);
    else CHECK(h == nullptr && has_message());
}

void null_handles() {
    float f = 0.f;
    int32_t i = 0;
    double ms[WENC_N_SITES];
    int64_t n[WENC_N_SITES];
    CHECK(wenc_load(nullptr, &f, 4) == WENC_EINVAL);
    CHECK(wenc_forward(nullptr, &f, 1, &f, nullptr) == WENC_EINVAL);
    CHECK(wenc_forward_ctx(nullptr, &f, 1, 500, &f, nullptr) == WENC_EINVAL);
    CHECK(wenc_forward_graph(nullptr, &f, 1, 1500, &f, nullptr) == WENC_EINVAL);
    CHECK(wenc_forward_tap(nullptr, &f, 1, 0, &f, nullptr) == WENC_EINVAL);
    CHECK(wenc_log_mel(nullptr, &f, 1, &f, nullptr) == WENC_EINVAL);
    CHECK(wenc_load_cross(nullptr, 1, &f, 4) == WENC_EINVAL);
    CHECK(wenc_prepare_cross(nullptr, &f, 1, 1500, &f, &f, nullptr) == WENC_EINVAL);
    CHECK(wenc_cross_attend(nullptr, &f, &f, &f, 1, 1, 1500, &f, nullptr) == WENC_EINVAL);
    CHECK(wenc_argmax(nullptr, &f, 1, 10, 10, &i, nullptr) == WENC_EINVAL);
    CHECK(wenc_profile(nullptr, 1) == WENC_EINVAL);
    CHECK(wenc_profile_read(nullptr, ms, n) == WENC_EINVAL);
    CHECK(has_message());
    wenc_destroy(nullptr);
    CHECK(wenc_last_error(nullptr) != nullptr);
}

void planner() {
    const int32_t Ms[] = {1, 15, 16, 255, 256, 257, 1504, 24000, 24064, 48000, (1 << 24) - 1};
    const int32_t Ns[] = {1, 4, 64, 384, 768, 1280, 2560, 3840, 5120, 1 << 20};
    const int32_t cus[] = {1, 32, 80, 256, 304, 1024};
    for (int32_t M : Ms)
        for (int32_t N : Ns)
            for (int32_t c : cus)
                for (int tile = -1; tile <= 1; ++tile)
                    for (int split = 0; split <= 1; ++split)
                        for (int streams = 1; streams <= 4; ++streams) {
                            int32_t big = -7;
                            const int kind = wenc_k_gemm_plan(M, N, c, tile, split, streams, &big);
                            CHECK(kind >= 0 && kind <= 2);
                            if (kind == 0) CHECK(big == 0);
                            if (kind == 1) CHECK(big == M);
                            if (kind == 2) CHECK(big > 0 && big < M && big % 256 == 0);
                        }
    int32_t big = 0;
    CHECK(wenc_k_gemm_plan(0, 64, 256, -1, 1, 1, &big) == WENC_EINVAL);
    CHECK(wenc_k_gemm_plan(64, -1, 256, -1, 1, 1, &big) == WENC_EINVAL);
    CHECK(wenc_k_gemm_plan(64, 64, 0, -1, 1, 1, &big) == WENC_EINVAL);
    CHECK(wenc_k_gemm_plan(64, 64, 256, 2, 1, 1, &big) == WENC_EINVAL);
    CHECK(wenc_k_gemm_plan(64, 64, 256, -1, 1, 0, &big) == WENC_EINVAL);
    CHECK(wenc_k_gemm_plan(64, 64, 256, -1, 1, 1, nullptr) == WENC_EINVAL);
    CHECK(wenc_k_gemm_mode(3, 1) == WENC_EINVAL && wenc_k_gemm_mode(-1, 5) == WENC_EINVAL);
    CHECK(wenc_k_gemm_mode(-1, 1) == WENC_OK);
}

void logmel_tables() {
    for (int nm = 8; nm <= 128; nm += 8) {
        int32_t nch = 0;
        CHECK(wenc_k_logmel_tables(nm, &nch, nullptr, nullptr, 0) == WENC_OK && nch >= 1 && 16 * nch <= 201);
        std::vector<int32_t> start(nm);
        std::vector<float> w(size_t(nm) * 16 * nch);
        CHECK(wenc_k_logmel_tables(nm, &nch, start.data(), w.data(), int64_t(w.size()) - 1) == WENC_EINVAL);
        CHECK(wenc_k_logmel_tables(nm, &nch, start.data(), w.data(), int64_t(w.size())) == WENC_OK);
        for (int m = 0; m < nm; ++m) {
            CHECK(start[m] >= 0 && start[m] + 16 * nch <= 201);
            bool any = false;
            for (int j = 0; j < 16 * nch; ++j) {
                const float x = w[size_t(m) * 16 * nch + j];
                CHECK(std::isfinite(x) && x >= 0.f);
                any = any || x > 0.f;
            }
            CHECK(any);  // every triangle of these banks covers at least one bin
        }
    }
    int32_t nch = 0;
    CHECK(wenc_k_logmel_tables(0, &nch, nullptr, nullptr, 0) == WENC_EINVAL);
    CHECK(wenc_k_logmel_tables(136, &nch, nullptr, nullptr, 0) == WENC_EINVAL);
    CHECK(wenc_k_logmel_tables(80, nullptr, nullptr, nullptr, 0) == WENC_EINVAL);
}

void kernel_arguments() {
    CHECK(wenc_k_gemm(nullptr, nullptr) == WENC_EINVAL);
    wenc_gemm_args a{};
    CHECK(wenc_k_gemm(&a, nullptr) == WENC_EINVAL);  // null operands
    const uint16_t buf[8] = {};
    const float fb[8] = {};
    a.A = buf;
    a.W = buf;
    a.bias = fb;
    a.M = 16;
    a.N = 16;
    a.K = 12;  // not a multiple of 8
    a.lda = a.ldw = 16;
    a.a_rows_per_batch = 16;
    CHECK(wenc_k_gemm(&a, nullptr) == WENC_EINVAL);
    a.K = 16;
    a.epilogue = 99;
    CHECK(wenc_k_gemm(&a, nullptr) == WENC_EINVAL);
    int32_t out = 0;
    float lg = 0.f;
    CHECK(wenc_argmax_noalloc(&lg, -1, 10, 10, &out, nullptr) == WENC_EINVAL);
    CHECK(wenc_argmax_noalloc(&lg, 1, 0, 10, &out, nullptr) == WENC_EINVAL);
    CHECK(wenc_argmax_noalloc(&lg, 1, 10, 9, &out, nullptr) == WENC_EINVAL);
    CHECK(wenc_argmax_noalloc(nullptr, 1, 10, 10, &out, nullptr) == WENC_EINVAL);
    CHECK(wenc_argmax_noalloc(&lg, 0, 10, 10, &out, nullptr) == WENC_OK);  // no rows: nothing to do
    CHECK(wenc_k_layernorm(fb, fb, fb, &out, -1, 64, 1e-5f, 0, nullptr) == WENC_EINVAL);
    CHECK(wenc_k_layernorm(fb, fb, fb, &out, 4, 66, 1e-5f, 0, nullptr) == WENC_EINVAL);
    CHECK(wenc_k_layernorm(nullptr, fb, fb, &out, 4, 64, 1e-5f, 0, nullptr) == WENC_EINVAL);
    CHECK(wenc_k_attention(buf, buf, buf, nullptr, 1, 1, 0, 64, nullptr) == WENC_EINVAL);
    CHECK(wenc_k_attention(buf, buf, buf, nullptr, 1, 1, 100, 100, nullptr) == WENC_EINVAL);
}

void messages_are_per_thread() {
    // a failure in one thread does not change the message another thread reads
    wenc_config bad = shape(80, 384, 4);
    bad.head_dim = 32;
    wenc_t *h = nullptr;
    CHECK(wenc_create(&bad, &h) == WENC_EINVAL);
    const std::string mine = wenc_last_error(nullptr);
    std::thread t([] {
        int32_t big = 0;
        (void)wenc_k_gemm_plan(0, 0, 0, 0, 0, 0, &big);
        const std::string theirs = wenc_last_error(nullptr);
        if (theirs.find("gemm plan") == std::string::npos) ++failures;
    });
    t.join();
    CHECK(mine == wenc_last_error(nullptr) && mine.find("head_dim") != std::string::npos);
}

}  // namespace

int main() {
    sizes_and_configs();
    null_handles();
    planner();
    logmel_tables();
    kernel_arguments();
    messages_are_per_thread();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
