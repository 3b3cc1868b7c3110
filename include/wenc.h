/*
 * wenc — the Whisper audio-encoder forward pass on one AMD Instinct MI355X
 * (gfx950), behind a plain C ABI.
 *
 * What is computed (whisper 0.9.0 API page, section model.nu; CKE page "How
 * Audio Becomes Words", the stitched-circuit figure):
 *
 *   mel [n_frames x n_mels] --conv1 (k3 s1 p1) + GELU--> [n_frames x d]
 *       --conv2 (k3 s2 p1) + GELU--> [n_ctx x d] --+ stored positions-->
 *   n_layer x [ x += out_proj(attn(LN1 x));  x += fc2(GELU(fc1(LN2 x))) ]
 *       --final LN--> out [n_ctx x d]
 *
 * attention is non-causal multi-head attention with scores q.k/sqrt(64)
 * (kernels.nu); k_proj has no bias (model.nu); GELU is the erf form
 * (kernels.nu); LayerNorm has a bias (kernels.nu).
 *
 * Conventions shared by every entry point:
 *   - Pointers named "device" are HIP device addresses owned by the caller
 *     (typically torch tensors); the library never frees them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Compute entry points only enqueue work on it and return without a host
 *     synchronisation.
 *   - Every int-returning call returns WENC_OK or a negative WENC_E* code;
 *     wenc_last_error() gives the message.  Argument errors are detected on
 *     the host before anything is enqueued.
 *   - A handle serves one stream at a time: two overlapping wenc_forward
 *     calls on one handle race on its scratch (one transcription at a time
 *     per device, as the whisper README's serving notes describe).
 */
#ifndef WENC_H
#define WENC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct wenc wenc_t;

/* Encoder shape.  Shapes are read from the checkpoint in the pages' design
 * (whisper README: nothing hardcoded to a model size); here the caller states
 * them.  Constraints checked by wenc_create:
 *   head_dim == 64, d_model == n_head * 64, n_mels % 8 == 0, d_ff % 8 == 0,
 *   n_frames even and == 2 * n_ctx, n_layer >= 0, 1 <= max_batch,
 *   max_batch * n_frames < 2^24, ln_eps > 0. */
typedef struct wenc_config {
    int32_t n_mels;     /* mel bins per frame (80; 128 for large-v3)          */
    int32_t d_model;    /* width                                               */
    int32_t n_head;     /* attention heads                                     */
    int32_t head_dim;   /* must be 64                                          */
    int32_t d_ff;       /* fc1 width (4 * d_model in Whisper)                  */
    int32_t n_layer;    /* encoder blocks                                      */
    int32_t n_frames;   /* mel frames per window (3000 for 30 s)               */
    int32_t n_ctx;      /* encoder positions = n_frames / 2 (1500)             */
    float   ln_eps;     /* LayerNorm epsilon (1e-5)                            */
    int32_t final_ln;   /* 1: apply the final LN (the encoder ends in one)     */
    int32_t max_batch;  /* windows per internal chunk; scratch is sized for it */
} wenc_config;

enum {
    WENC_OK = 0,
    WENC_EINVAL = -1, /* bad argument: config, size, null pointer, batch < 0 */
    WENC_ENOMEM = -2, /* device allocation failed; message has bytes asked and free */
    WENC_ENODEV = -3, /* no HIP device, or the device is not gfx950            */
    WENC_ESTATE = -4, /* forward before wenc_load                              */
    WENC_EHIP = -5    /* HIP runtime or launch error; message has its string   */
};

/* Validate `cfg`, allocate the device weight arena and the activation
 * scratch for cfg->max_batch windows on the current HIP device.  On success
 * *out owns them; on failure *out is NULL and wenc_last_error(NULL) explains
 * (the whisper README's implementation notes: a failed device allocation is
 * reported with the device's memory, never run past). */
int wenc_create(const wenc_config *cfg, wenc_t **out);

/* Exact byte size of the canonical weight blob for `cfg`, 0 if invalid.
 * Blob: IEEE binary16, little-endian, in the field order of the Whisper
 * struct on the whisper 0.9.0 API page (model.nu):
 *   conv1_w [d][n_mels][3], conv1_b [d], conv2_w [d][d][3], conv2_b [d],
 *   pos [n_ctx][d],
 *   per layer: ln1_g [d], ln1_b [d], wq [d][d], bq [d], wk [d][d] (no bias
 *   entry: k_proj has none), wv [d][d], bv [d], wo [d][d], bo [d],
 *   ln2_g [d], ln2_b [d], fc1_w [d_ff][d], fc1_b [d_ff], fc2_w [d][d_ff],
 *   fc2_b [d],
 *   lnf_g [d], lnf_b [d].
 * Matrices are [out][in] row-major (kernels.nu, wk_matvec: W[rows][cols]). */
size_t wenc_weights_nbytes(const wenc_config *cfg);

/* Copy a HOST blob (layout above) into the device arena, repacking it once
 * (conv taps to [out][k][in], q|k|v concatenated with a zero k bias, gains,
 * biases and positions widened exactly to fp32) in one upload.  The blob is
 * read for the upload and not retained, and the matrix weights stay fp16 on
 * the device (whisper README, "Performance and memory": the checkpoint is
 * mapped for the upload and released, f16 weights stay f16; whisper 0.9.0
 * API page, wh_open: one device arena per model, freed as a whole).
 * nbytes must equal wenc_weights_nbytes, else WENC_EINVAL with nothing
 * changed.  Synchronous.  May be called again to replace the weights: it
 * first waits for all work already enqueued on the device (on any stream)
 * to finish, so a forward still in flight reads the old weights to its
 * end.  If the upload fails (WENC_EHIP) the handle counts as not loaded
 * and wenc_forward returns WENC_ESTATE until a later wenc_load succeeds
 * (whisper README, "Implementation notes": a failure is reported, never
 * run past). */
int wenc_load(wenc_t *h, const void *blob, size_t nbytes);

/* out[b] = encoder(mel[b]) for b < batch.
 *   mel: device, fp32 [batch][n_frames][n_mels], a frame contiguous
 *        (whisper 0.9.0 API page, wh_encode); 16-byte aligned.
 *   out: device, fp32 [batch][n_ctx][d_model] row-major (wh_enc_out);
 *        16-byte aligned.
 * batch == 0 is a no-op; batch > max_batch runs in chunks of max_batch.
 * WENC_EINVAL (before any launch) for a NULL or misaligned pointer or
 * batch < 0; WENC_ESTATE before a successful wenc_load.
 * Enqueued on `stream`; no host synchronisation. */
int wenc_forward(wenc_t *h, const float *mel, int32_t batch, float *out, void *stream);

/* Shortened-context forward (drafts; whisper README, section Serving:
 * a draft encodes the audio plus 5 s, at least 10 s, instead of the full
 * 30 s window, as whisper.cpp's audio_ctx does).  The same encoder runs over
 * 2 * n_ctx frames and adds the FIRST n_ctx rows of the stored position
 * table; attention spans those n_ctx positions only.
 *   mel: device, fp32 [batch][2 * n_ctx][n_mels], 16-byte aligned;
 *   out: device, fp32 [batch][n_ctx][d_model], 16-byte aligned.
 * 1 <= n_ctx <= the configured n_ctx, else WENC_EINVAL before any launch
 * (as for a NULL or misaligned pointer);
 * n_ctx equal to the configured one is wenc_forward.  Windows are chunked by
 * what the scratch holds at this length (more than max_batch when n_ctx is
 * shorter).  Enqueued on `stream`; no host synchronisation. */
int wenc_forward_ctx(wenc_t *h, const float *mel, int32_t batch, int32_t n_ctx, float *out, void *stream);

/* Record once, replay: the same forward as wenc_forward_ctx (n_ctx equal to
 * the configured one is a full window), enqueued as one recorded HIP graph
 * (whisper README, "Implementation notes": the encoder is recorded once
 * and replayed).  The first call with a given (mel, out, batch, n_ctx)
 * records every launch of the forward, chunks and both stream groups
 * included, into a graph on a stream the handle owns and instantiates it;
 * that call and every later call with the same four values launch the
 * graph on `stream`.  A call with any other value records anew and
 * replaces the kept graph.  The graph refers to the handle's weight arena
 * and scratch by address: it stays valid across wenc_load (which rewrites
 * the arena in place) and is released by wenc_destroy.  Same arguments,
 * alignment and errors as wenc_forward_ctx; WENC_ESTATE while per-launch
 * profiling (wenc_profile) or WENC_DEBUG_SYNC is on, which a graph cannot
 * hold.  One stream at a time per handle, as for every forward. */
int wenc_forward_graph(wenc_t *h, const float *mel, int32_t batch, int32_t n_ctx, float *out, void *stream);

/* Release the handle and every device allocation it owns (whisper 0.9.0
 * API page, wh_close, and the Whisper struct's list of every device
 * allocation kept for the free).  NULL-safe.  Synchronises the device first
 * so no enqueued work still uses the memory.  The handle must not be used
 * afterwards. */
void wenc_destroy(wenc_t *h);

/* Message for the last failure on `h` (or of wenc_create / handle-less calls
 * in this thread when h is NULL): the library's failures come back as a
 * status code plus a message, as wh_open on the whisper 0.9.0 API page
 * returns either the model or an error string.  Never NULL; "" when there
 * is none.  The pointer stays valid until the next failing call on the
 * same handle (or, for h == NULL, in the same thread). */
const char *wenc_last_error(const wenc_t *h);

/* Log-mel spectrogram of whole windows, the encoder's input (CKE page, "The
 * Frontend: Sound Becomes A Tensor"): STFT power with n_fft 400, hop 160, a
 * periodic Hann window and reflect padding (frames centred, the last STFT
 * frame dropped); n_mels area-normalised triangles on the Slaney mel scale
 * over 0 .. 8 kHz; log10 of max(power, 1e-10); clamp at the window's maximum
 * minus 8 (-80 dB); (x + 4) / 4.  All in fp32; the STFT is the 20 x 20
 * mixed-radix FFT of the same section.
 *   audio: device fp32 [batch][160 * n_frames], 16 kHz mono, already padded
 *          or cut to the window (480,000 samples for 3000 frames); 4-byte
 *          aligned;
 *   mel:   device fp32 [batch][n_frames][n_mels], wenc_forward's input;
 *          16-byte aligned (else WENC_EINVAL before any launch).
 * Needs n_mels a multiple of 8, <= 128 (Whisper uses 80 and 128), else
 * WENC_EINVAL.  batch > max_batch runs in chunks.  Enqueued on `stream`. */
int wenc_log_mel(wenc_t *h, const float *audio, int32_t batch, float *mel, void *stream);

/* ------------------------------------------------------------------------
 * Cross-attention K/V of the decoder, projected from the encoder memory once
 * per clip (whisper 0.9.0 API page, wh_prepare_cross: the encoder does not
 * change while a clip is transcribed, so its K and V are not recomputed per
 * token; model.nu: per decoder layer x_wk has no bias, x_wv has x_bv).
 * ---------------------------------------------------------------------- */

/* Byte size of the cross-attention blob for n_dec_layer decoder layers of
 * width d_model: per layer, in this order, x_wk [d][d], x_wv [d][d], x_bv [d],
 * all fp16 (IEEE binary16, little-endian), matrices [out][in] row-major.
 * 0 for an invalid config or n_dec_layer <= 0. */
size_t wenc_cross_nbytes(const wenc_config *cfg, int32_t n_dec_layer);

/* Copy a HOST cross blob into a device arena of the handle (replacing any
 * earlier one), stacked per layer as [x_wk; x_wv] fp16 [2d][d] with bias
 * [0; x_bv] fp32.  nbytes must equal wenc_cross_nbytes.  Synchronous. */
int wenc_load_cross(wenc_t *h, int32_t n_dec_layer, const void *blob, size_t nbytes);

/* For every loaded decoder layer l and window b < batch:
 *   xk[l][b] = memory[b] . x_wk[l]^T,  xv[l][b] = memory[b] . x_wv[l]^T + x_bv[l].
 *   memory: device fp32 [batch][n_ctx][d_model] (wenc_forward's or
 *           wenc_forward_ctx's out), rounded to fp16 once before use;
 *   xk, xv: device fp16 [n_dec_layer][batch][n_ctx][d_model] each;
 *   all three 16-byte aligned (else WENC_EINVAL before any launch).
 * 1 <= n_ctx <= the configured n_ctx.  WENC_ESTATE before wenc_load_cross.
 * Uses the handle's scratch (no forward may overlap it).  Enqueued on
 * `stream`; no host synchronisation. */
int wenc_prepare_cross(wenc_t *h, const float *memory, int32_t batch, int32_t n_ctx, void *xk, void *xv,
                       void *stream);

/* ------------------------------------------------------------------------
 * Stage taps and kernel entry points.  They expose each step of the path in
 * isolation so that it can be compared with an independent implementation
 * (the CKE page: every kernel has its own parity oracle).  All pointers are
 * device pointers; fp16 buffers are IEEE binary16 bit patterns (uint16_t).
 * ---------------------------------------------------------------------- */

/* Stage taps of wenc_forward (batch <= max_batch):
 *   WENC_TAP_C1:    dst fp16 [batch][n_frames][d]   conv1 + GELU
 *   WENC_TAP_STEM:  dst fp32 [batch][n_ctx][d]      conv2 + GELU + positions
 *   WENC_TAP_BLOCK + l: dst fp32 [batch][n_ctx][d]  residual after block l  */
enum { WENC_TAP_C1 = 0, WENC_TAP_STEM = 1, WENC_TAP_BLOCK = 2 };
int wenc_forward_tap(wenc_t *h, const float *mel, int32_t batch, int32_t tap, void *dst, void *stream);

/* LayerNorm over rows of x (kernels.nu: mean-subtracting, with bias):
 *   y[r][i] = (x[r][i] - mean_r) / sqrt(var_r + eps) * gamma[i] + beta[i],
 * population variance.  x fp32 [rows][d]; gamma, beta fp32 [d];
 * y fp32 (out_f32 = 1) or fp16 [rows][d].  d % 4 == 0, d <= 2048. */
int wenc_k_layernorm(const float *x, const float *gamma, const float *beta, void *y,
                     int32_t rows, int32_t d, float eps, int32_t out_f32, void *stream);

/* Epilogues of the fp16 MFMA GEMM  acc[m][n] = sum_k A[m][k] * W[n][k]. */
enum {
    WENC_EPI_GELU_F16 = 0, /* C fp16 = gelu(acc + bias)                       (fc1, conv1) */
    WENC_EPI_CONV2 = 1,    /* C fp32 = gelu(acc + bias) + pos[m % pos_rows]   (conv2)      */
    WENC_EPI_RESID = 2,    /* C fp32 += acc + bias                            (out_proj, fc2) */
    WENC_EPI_QKV = 3,      /* q, k, v^T scatter, see wenc_gemm_args           (qkv)        */
    WENC_EPI_KV = 4        /* C, C2 fp16 = acc + bias, split at n_split       (cross K/V)  */
};

/* GEMM arguments.  Row m of A starts at
 *   A + (m / a_rows_per_batch) * a_batch_stride + (m % a_rows_per_batch) * lda
 * (elements), which expresses both plain row-major A (a_rows_per_batch = M,
 * lda = K) and the conv stem's overlapping frame windows over a zero-padded,
 * frame-contiguous input (lda = stride * C_in, K = 3 * C_in).  W is
 * [N][ldw] row-major fp16 (K contiguous).  Output row m of C starts at
 *   C + (m / c_rows_per_batch) * c_batch_stride
 *     + (m % c_rows_per_batch + c_row_offset) * ldc.
 * QKV: N = 3 * n_head * 64; columns [0, d) go to q and [d, 2d) to k as
 * [batch][n_head][T][64] fp16, columns [2d, 3d) to vt as
 * [batch][n_head][64][ldvt] fp16 with m = b * T + t, where key t of a row
 * sits at slot t with bits 2 and 3 swapped (the order the attention kernel
 * consumes) and the slots of keys T .. ldvt-1 are written with zeros; the q
 * slice is multiplied by q_scale after its bias.
 * KV: columns [0, n_split) go to C and [n_split, N) to C2 (column
 * n - n_split), both fp16 with row m at m * ldc; 0 < n_split <= N,
 * n_split % 4 == 0, ldc >= max(n_split, N - n_split).  Requires K % 8 == 0,
 * lda % 8 == 0, ldw % 8 == 0, a_batch_stride % 8 == 0, N, ldc and
 * c_batch_stride multiples of 4, ldvt a multiple of 64, M < 2^24. */
typedef struct wenc_gemm_args {
    const uint16_t *A; int64_t a_batch_stride; int32_t a_rows_per_batch; int32_t lda;
    const uint16_t *W; int32_t ldw;
    const float *bias;           /* [N] fp32, never NULL                        */
    void *C; int64_t c_batch_stride; int32_t c_rows_per_batch; int32_t c_row_offset; int32_t ldc;
    const float *pos; int32_t pos_rows;   /* CONV2 only: fp32 [pos_rows][N]     */
    uint16_t *q; uint16_t *k; uint16_t *vt; int32_t T; int32_t n_head; int32_t ldvt; float q_scale;
    int32_t M, N, K;
    int32_t epilogue;
    uint16_t *C2; int32_t n_split;        /* KV only                            */
} wenc_gemm_args;
int wenc_k_gemm(const wenc_gemm_args *args, void *stream);

/* Decode-step cross-attention over one decoder layer's cached K/V: the
 * attention a generated token runs over the n_ctx encoder positions (whisper
 * README, "Performance and memory": one query, the keys split across
 * blocks and the partial softmaxes merged; whisper 0.9.0 API page,
 * wh_prepare_cross: per layer xk, xv of n_ctx x d_model; kernels.nu:
 * scores q.k / sqrt(64)).  For batch item b, query row i and head h
 * (columns [64h, 64h + 64)):
 *   out[b][i][h] = sum_u softmax_u(q[b][i][h] . xk[b][u][h] / 8) xv[b][u][h]
 * over u < n_ctx, no mask.  q, out: device fp16 [batch][n_q][d_model]
 * (q after q_proj); xk, xv: device fp16 [batch][n_ctx][d_model], e.g. one
 * decoder layer's slice of wenc_prepare_cross's output; all four 16-byte
 * aligned, caller-owned.  1 <= n_q <= 8 (queries per sequence: one for
 * greedy decoding, a few for beams), 1 <= n_ctx <= cfg.n_ctx, batch >= 0
 * (chunked through the handle's activation scratch, which it shares with
 * wenc_forward: one call at a time per handle).  Scores, probabilities and
 * sums are fp32; out is rounded to fp16 once.  Deterministic, and an item's
 * output bits do not depend on the batch it is computed in (the library
 * picks one launch or two by the batch's size; both sum in the same order).
 * Enqueues on `stream`, no host sync.  EINVAL for bad sizes, NULL or
 * misaligned pointers. */
int wenc_cross_attend(wenc_t *h, const void *q, const void *xk, const void *xv, int32_t batch, int32_t n_q,
                      int32_t n_ctx, void *out, void *stream);

/* Greedy token choice on the device: per row, the index of the largest
 * logit, so that a decode step returns one integer per sequence instead of
 * the whole vocabulary (whisper README, "Performance and memory": greedy
 * decoding's argmax over the 51865 logits, reduced on the device).
 *   out[r] = min { i : logits[r][i] = max_j logits[r][j] }
 * Ties go to the smallest index; -0.0 equals +0.0; a NaN counts as larger
 * than every number (the first NaN wins).  logits: device fp32
 * [rows][ld] (row r at logits + r * ld), out: device int32 [rows]; both
 * 4-byte aligned, caller-owned.  1 <= n_vocab <= 2^30, ld >= n_vocab,
 * rows >= 0 (the per-chunk keys go to the handle's activation scratch,
 * which it shares with wenc_forward: one call at a time per handle).
 * Exact: no arithmetic, only comparisons.  Enqueues on `stream`, no host
 * sync.  EINVAL for bad sizes, NULL or misaligned pointers. */
int wenc_argmax(wenc_t *h, const float *logits, int32_t rows, int32_t n_vocab, int64_t ld, int32_t *out,
                void *stream);

/* wenc_argmax without a handle and without allocating: for callers that
 * cannot allocate device memory (code being recorded into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc).  Same result, arguments
 * and error behaviour as wenc_argmax, whose kernels it runs; the per-chunk
 * keys go to a 1 MiB array of 131072 keys that the library's code object
 * holds on each device (kept until the process ends) instead of a handle's
 * scratch, in passes of 131072 / ceil(n_vocab / 2048) rows.  No hipMalloc,
 * hipFree or other allocating call is made.  Limit: ceil(n_vocab / 2048) <=
 * 131072 (n_vocab <= 268435456), else WENC_EINVAL before any launch.  Every
 * call on one device shares that device's array: calls that overlap on one
 * device (on different streams or threads) race and may return wrong
 * indices; calls in one stream's order are safe.  Errors are reported
 * through wenc_last_error(NULL). */
int wenc_argmax_noalloc(const float *logits, int32_t rows, int32_t n_vocab, int64_t ld, int32_t *out,
                        void *stream);

/* Test-only: the tile configuration of every later GEMM launch in this
 * process (all handles).  tile: -1 automatic (the default, or the
 * WENC_GEMM_TILE environment variable when set), 0 = 128 x 128 tiles,
 * 1 = 256 x 256 tiles, 2 = 256 x 256 tiles whose main loop runs every wave
 * in the same phase (the default 256 x 256 main loop runs the two waves of
 * a SIMD a phase apart, one issuing MFMAs while the other reads LDS).
 * split: 1 (the default) lets an automatic launch give
 * its last 256-row tile rows to 128 x 128 tiles when that evens out the last
 * round over the compute units, 0 keeps one tile size.  Every configuration
 * sums each output over k in the same order, so all give the same bits.
 * The two values are stored atomically: a launch on another thread sees
 * each one either before or after the change (so it may pair a new tile
 * with an old split).  Returns WENC_EINVAL for values out of range. */
int wenc_k_gemm_mode(int32_t tile, int32_t split);

/* Test-only, host logic (no device work): the tile plan a GEMM launch uses
 * for M output rows (after the QKV epilogue's padding to 16 keys per item)
 * and N columns on a device of `cus` compute units, with tile and split as
 * in wenc_k_gemm_mode (tile -1 = automatic, ignoring the environment), when
 * `streams` streams run such launches side by side (1 for wenc_k_gemm and a
 * forward kept on one stream, 2 for wenc_forward's default split).  Returns
 * 0 = all 128 x 128 tiles, 1 = all 256 x 256 tiles, 2 = 256 x 256 tiles for
 * rows [0, *big_rows) and 128 x 128 for the rest; *big_rows is M for 1 and
 * 0 for 0.  WENC_EINVAL for values out of range. */
int wenc_k_gemm_plan(int32_t M, int32_t N, int32_t cus, int32_t tile, int32_t split, int32_t streams,
                     int32_t *big_rows);

/* Test-only, host logic (no device work): the mel-filter tables wenc_log_mel
 * reads for n_mels filters (CKE page, "The Frontend": area-normalised
 * triangles on the Slaney scale over 0 .. 8 kHz at the 201 bins k * 40 Hz).
 * Filter m is a window of 16 * (*nch) bins starting at mstart[m], inside bins
 * 0 .. 200, whose weights are mwt[m][0 .. 16 nch), zero outside the
 * triangle.  Writes *nch; fills mstart [n_mels] and mwt (row-major, capacity
 * mwt_cap floats) when both are non-NULL.  WENC_EINVAL when wenc_log_mel
 * would refuse n_mels (not a multiple of 8 in 8 .. 128), nch is NULL or
 * mwt_cap is too small. */
int wenc_k_logmel_tables(int32_t n_mels, int32_t *nch, int32_t *mstart, float *mwt, int64_t mwt_cap);

/* Non-causal attention per (batch, head) (kernels.nu, wk_attn with causal 0):
 *   ao[b][t][h*64 + e] = sum_u softmax_u(q[b][h][t] . k[b][h][u]) * v[b][h][u][e]
 * with q ALREADY scaled by log2(e)/sqrt(64) (the softmax is taken in base 2),
 * q, k fp16 [batch][n_head][T][64], ao fp16 [batch][T][n_head*64], and v
 * given transposed as vt fp16 [batch][n_head][64][ldvt] in the key-slot
 * order the QKV epilogue writes (key u at slot u with bits 2 and 3 swapped);
 * slots of keys T .. ldvt-1 must hold finite values.  ldvt % 64 == 0,
 * ldvt >= T. */
int wenc_k_attention(const uint16_t *q, const uint16_t *k, const uint16_t *vt, uint16_t *ao,
                     int32_t batch, int32_t n_head, int32_t T, int32_t ldvt, void *stream);

/* Per-launch timing of wenc_forward, wenc_forward_ctx, wenc_prepare_cross,
 * wenc_log_mel, wenc_cross_attend and wenc_argmax: HIP events recorded
 * around every launch whose site bit is set in `site_mask` (bit s =
 * 1 << WENC_SITE_*), on the stream that launch goes to (the caller's, or
 * the handle's second stream for the second window group of a forward);
 * 0 turns it off.  Events are read, and cleared, by wenc_profile_read
 * (which synchronises on them).  While a mask is set wenc_forward_graph
 * refuses to record. */
enum {
    WENC_SITE_INGEST = 0, WENC_SITE_CONV1 = 1, WENC_SITE_CONV2 = 2, WENC_SITE_LN1 = 3,
    WENC_SITE_QKV = 4, WENC_SITE_ATTN = 5, WENC_SITE_OPROJ = 6, WENC_SITE_LN2 = 7,
    WENC_SITE_FC1 = 8, WENC_SITE_FC2 = 9, WENC_SITE_LNF = 10, WENC_SITE_XCVT = 11,
    WENC_SITE_XKV = 12, WENC_SITE_MEL = 13, WENC_SITE_XATT = 14, WENC_SITE_ARGMAX = 15,
    WENC_N_SITES = 16
};
int wenc_profile(wenc_t *h, uint32_t site_mask);
/* ms_total[s] and launches[s] for s < WENC_N_SITES (arrays of that length):
 * launches[s] counts the recorded launches of site s, and ms_total[s] is the
 * time during which at least one of them was running (the length of the
 * union of their intervals, so launches of one site that overlap on the
 * streams of a split forward count once; on one stream it is the sum). */
int wenc_profile_read(wenc_t *h, double *ms_total, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* WENC_H */
