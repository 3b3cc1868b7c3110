// Host-side launchers of the gfx950 kernels (internal to libwenc.so).
#pragma once

#include <hip/hip_runtime.h>
#include "wenc.h"

namespace wk {

// Checks the shape/alignment contract of wenc_gemm_args; returns a message
// or nullptr when the arguments are acceptable.
const char *gemm_check(const wenc_gemm_args &a);
// tag 1 selects a separately named copy of the kernel (fc1, fc2); the tile
// plan is made for the device's compute units divided by cu_div (the share
// of one stream when two streams run GEMMs side by side).
hipError_t launch_gemm(const wenc_gemm_args &a, hipStream_t s, int tag = 0, int cu_div = 1);
// Tile configuration of later launches (see wenc_k_gemm_mode); -1 if out of range.
int gemm_mode(int tile, int split);
// Tile plan of one GEMM launch over M rows (as the kernel sees them) and N
// columns on a device of `cus` compute units shared by `streams` streams
// running launches side by side: all 128 x 128 tiles, all 256 x 256, or
// 256 x 256 for rows [0, big_rows) and 128 x 128 for the rest.  tile: -1
// chooses, 0 / 1 force 128 / 256; split 0 keeps one tile size.
enum { GEMM_PLAN_SMALL = 0, GEMM_PLAN_BIG = 1, GEMM_PLAN_SPLIT = 2 };
struct GemmPlan {
    int kind;
    int big_rows;
};
GemmPlan gemm_plan(int M, int N, long cus, int tile, int split, int streams);

const char *attention_check(int batch, int n_head, int T, int ldvt);
hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *vt, uint16_t *ao,
                            int batch, int n_head, int T, int ldvt, hipStream_t s);

const char *layernorm_check(int rows, int d);
hipError_t launch_layernorm(const float *x, const float *g, const float *b, void *y, int rows, int d,
                            float eps, bool out_f32, hipStream_t s);

// mel fp32 [B][F][nm] -> melp fp16 [B][F+2][nm] with zero first/last frame,
// and zero rows 0 and F+1 of c1 fp16 [B][F+2][d].
hipError_t launch_ingest(const float *mel, uint16_t *melp, uint16_t *c1, int B, int F, int nm, int d,
                         hipStream_t s);

// Log-mel frontend: audio fp32 [batch][160 n_frames] -> out fp32
// [batch][n_frames][n_mels].  tab: [400] (cos, -sin) pairs of 2 pi i / 400;
// win: [400] periodic Hann; filter m's weights at bins mstart[m] .. mstart[m]
// + 16 nch - 1 are mwt[m][0 .. 16 nch) (16-byte aligned rows, zero outside
// the triangle, mstart[m] + 16 nch <= 201); blkmax: [batch][tiles].
constexpr int LOGMEL_MAX_MELS = 128;
constexpr int LOGMEL_MAX_EXTRA = 1024;  // n_mels (nch - 1) 16: the weights past each filter's first 16 bins
int logmel_tiles(int n_frames);
const char *logmel_check(int batch, int n_frames, int n_mels);
hipError_t launch_logmel(const float *audio, int batch, int n_frames, const float *tab, const float *win,
                         const float *mwt, const int *mstart, int nch, int n_mels, float *out, float *blkmax,
                         hipStream_t s);

// Compute units of the current device (cached per device).
long cu_count();

// Decode-step cross-attention (xattn.hip): q fp16 [batch][n_q][64 n_head],
// xk, xv fp16 [batch][T][64 n_head] (16-byte aligned), out fp16 like q;
// part: fp32 workspace of xattn_part_bytes(batch, n_head, n_q, T) bytes.
constexpr int XATTN_MAX_Q = 8;
size_t xattn_part_bytes(int batch, int n_head, int n_q, int T);
const char *xattn_check(int batch, int n_head, int n_q, int T);
hipError_t launch_xattn(const uint16_t *q, const uint16_t *xk, const uint16_t *xv, uint16_t *out, float *part,
                        int batch, int n_head, int n_q, int T, hipStream_t s);

// Greedy argmax per row (argmax.hip): logits fp32 [rows][ld], out int32
// [rows]; part: workspace of rows * argmax_chunks(n_vocab) keys (unused when
// that is one chunk per row).
int argmax_chunks(int n_vocab);
// The allocation-free variant's chunk keys: a file-scope device array of
// ARGMAX_STATIC_KEYS keys (1 MiB) per device.  static_scratch() gives its
// address on the current device (looked up on the first call per device).
constexpr int64_t ARGMAX_STATIC_KEYS = int64_t(1) << 17;
hipError_t static_scratch(uint64_t **keys);
const char *argmax_check(int rows, int n_vocab, int64_t ld);
hipError_t launch_argmax(const float *logits, int rows, int n_vocab, int64_t ld, uint64_t *part, int32_t *out,
                         hipStream_t s);

// y fp16 [n] = x fp32 [n] rounded to nearest even; n % 4 == 0, 16-byte aligned.
hipError_t launch_to_f16(const float *x, uint16_t *y, int64_t n, hipStream_t s);

}  // namespace wk
