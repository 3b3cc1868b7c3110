"""Throughput of the Whisper audio-encoder forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

A step is one wenc_forward over one batch of synthetic windows (conv stem,
all blocks, final LN), with the mel input and the weights already resident
in device memory.  Prints ONE JSON line.  Per-launch kernel times come from
HIP events the library records on the same stream around each launch of the
dominant kernel during the timed steps; the fp64 oracle is timed on the
host on a bounded sample for the cpu_baseline field.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "encoder 30s-windows/sec and TFLOP/s (% of fp16 MFMA peak), 1 MI355X"
PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
N_VOCAB = 51865            # Whisper's vocabulary: the logits a greedy decode step reduces


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def site_work(cfg, B):
    """Algorithmic FLOPs (MFMA sites) or HBM bytes (memory-bound sites) of one launch."""
    T, F, d, nm, H, Fd = cfg.n_ctx, cfg.n_frames, cfg.d_model, cfg.n_mels, cfg.n_head, cfg.d_ff
    M = B * T
    return {
        "conv1": ("mfma", 2.0 * B * F * d * 3 * nm),
        "conv2": ("mfma", 2.0 * M * d * 3 * d),
        "qkv": ("mfma", 2.0 * M * 3 * d * d),
        "attn": ("mfma", 4.0 * B * H * T * T * 64),
        "oproj": ("mfma", 2.0 * M * d * d),
        "fc1": ("mfma", 2.0 * M * Fd * d),
        "fc2": ("mfma", 2.0 * M * d * Fd),
        # LN: read fp32 x, write fp16 (final: fp32); gains and biases are negligible
        "ln1": ("hbm", M * d * (4.0 + 2.0)),
        "ln2": ("hbm", M * d * (4.0 + 2.0)),
        "lnf": ("hbm", M * d * (4.0 + 4.0)),
        "ingest": ("hbm", B * F * nm * 4.0 + B * (F + 2) * nm * 2.0),
        # cross K/V, per decoder layer: [B T, d] x [d, 2d]; the conversion reads fp32, writes fp16
        "xkv": ("mfma", 2.0 * M * 2 * d * d),
        "xcvt": ("hbm", M * d * (4.0 + 2.0)),
        # log-mel: per frame, the 20 x 20 FFT with the window and the power as the kernel evaluates it
        "mel": ("alu", B * F * FFT_FLOPS_PER_FRAME),
        # decode-step cross-attention, per decoder layer: K and V read once (fp16)
        "xatt": ("hbm", 2.0 * M * d * 2.0),
        # greedy argmax of a decode step: one row of N_VOCAB fp32 logits per window, read once
        "amax": ("hbm", B * N_VOCAB * 4.0),
    }


PROFILES = os.path.join(HERE, "profiles")
CSRC = "whisper_audio_encoder_amd/csrc/"
SITE_SOURCES = {"attn": ("attention.hip", "common.h"), "ln1": ("layernorm.hip", "common.h"),
                "ln2": ("layernorm.hip", "common.h"), "lnf": ("layernorm.hip", "common.h"),
                "ingest": ("layernorm.hip", "common.h"), "xcvt": ("layernorm.hip", "common.h")}


def kernel_source_hash(site):
    """sha256 over the sources of the kernel a site launches."""
    import hashlib
    h = hashlib.sha256()
    for f in SITE_SOURCES.get(site, ("gemm.hip", "common.h")):
        with open(os.path.join(HERE, CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, site):
    """HBM bytes per launch of `site` from the committed PMC summary, or None
    when there is none or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{site}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_sha256") != kernel_source_hash(site):
        return None
    return t.get("hbm_bytes_per_launch")


def gemm_tile_costs(steps=20):
    """Per-tile cost of the 256 x 256 GEMM kernel: M = 16384, N = 4096 (1024
    tiles, four rounds of one tile per compute unit on 256 CUs), K from 64 to
    2048, with the fp16 GELU epilogue and the fp32 residual epilogue.  A
    line fitted to the time per round against the k steps (K >= 256) splits
    it into a cost per 64-wide k step and a fixed cost per tile (prologue and
    epilogue).  The same again under light load: M = 1024, N = 2048 (32
    tiles, one round on 32 compute units, the rest of the chip idle).
    Prints one JSON line."""
    import numpy as np
    import torch
    from whisper_audio_encoder_amd import wenc
    if wenc.lib().wenc_k_gemm_mode(1, 0) != wenc.WENC_OK:  # 256 x 256 tiles everywhere, no tail split
        raise RuntimeError(wenc.wenc_last_error())
    out = {}

    def series(M, N, epi, rounds):
        pts = []
        for K in (64, 128, 256, 512, 1024, 2048):
            A = torch.randn(M, K, device="cuda:0").half()
            W = (0.02 * torch.randn(N, K, device="cuda:0")).half()
            b = torch.zeros(N, device="cuda:0")
            C = (torch.empty(M, N, device="cuda:0", dtype=torch.half) if epi == wenc.WENC_EPI_GELU_F16
                 else torch.zeros(M, N, device="cuda:0"))
            g = wenc.wenc_gemm_args()
            g.A, g.W, g.bias, g.C = A.data_ptr(), W.data_ptr(), b.data_ptr(), C.data_ptr()
            g.a_rows_per_batch, g.lda, g.ldw = M, K, K
            g.c_rows_per_batch, g.ldc = M, N
            g.M, g.N, g.K, g.epilogue = M, N, K, epi
            for _ in range(3):
                wenc.wenc_k_gemm(g)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                wenc.wenc_k_gemm(g)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            pts.append({"K": K, "us_per_launch": round(us, 2), "us_per_round": round(us / rounds, 3)})
        x = np.array([p["K"] // 64 for p in pts[2:]], float)
        y = np.array([p["us_per_round"] for p in pts[2:]])
        step_us, fixed_us = np.polyfit(x, y, 1)
        return {"points": pts, "us_per_k_step": round(float(step_us), 3), "us_fixed_per_tile": round(float(fixed_us), 2)}

    try:
        for M, N, sfx in ((16384, 4096, ""), (1024, 2048, "_32_tiles")):
            tiles = M // 256 * (N // 256)
            rounds = max(1.0, tiles / 256)
            out["shape" + sfx] = {"M": M, "N": N, "tiles": tiles, "rounds_on_256_cus": rounds}
            out["gelu_f16" + sfx] = series(M, N, wenc.WENC_EPI_GELU_F16, rounds)
            out["residual_f32" + sfx] = series(M, N, wenc.WENC_EPI_RESID, rounds)
    finally:
        wenc.lib().wenc_k_gemm_mode(-1, 1)
    print(json.dumps(out), flush=True)


def copy_probe(nbytes):
    """A plain device-to-device copy of known size (calibrates the HBM byte counters)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 5}), flush=True)


def hbm_ceiling(steps=50):
    """The LayerNorm against plain conversions that move the same bytes: per
    shape (24000 x 1280 and 24000 x 768, the encoder's rows at d 1280 and
    768), an fp32 -> fp16 conversion by torch (reads 4 and writes 2 bytes per
    element, as the LayerNorm does), an fp32 copy of the same number of
    bytes moved, and the library's LayerNorm.  Prints one JSON line of
    achieved GB/s (bytes read + written over the average launch time)."""
    import torch
    from whisper_audio_encoder_amd import wenc

    def rate(fn, nbytes):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        return {"us": round(us, 2), "GB_per_s": round(nbytes / us / 1e3, 1)}

    out = {}
    g = torch.Generator(device="cuda:0").manual_seed(5)
    for rows, d in ((24000, 1280), (24000, 768)):
        n = rows * d
        x = torch.randn(rows, d, device="cuda:0", generator=g)
        y16 = torch.empty(rows, d, device="cuda:0", dtype=torch.half)
        gam = torch.ones(d, device="cuda:0")
        bet = torch.zeros(d, device="cuda:0")
        c_src = torch.empty(n * 6 // 8, device="cuda:0")  # fp32 copy moving 6 bytes per element
        c_dst = torch.empty_like(c_src)
        out[f"{rows}x{d}"] = {
            "bytes": 6 * n,
            "torch_fp32_to_fp16": rate(lambda: y16.copy_(x), 6 * n),
            "torch_fp32_copy": rate(lambda: c_dst.copy_(c_src), 6 * n),
            "layernorm": rate(lambda: wenc.wenc_k_layernorm(x, gam, bet, y16, rows, d, 1e-5, False,
                                                            torch.cuda.current_stream()), 6 * n),
        }
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, mel, params, budget_s=30.0):
    """Time the fp64 oracle on one window of the workload (all blocks)."""
    import oracle
    from threadpoolctl import threadpool_info
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t0 = time.perf_counter()
    oracle.encode(mel[0], params, cfg.n_layer, cfg.n_head, cfg.ln_eps, bool(cfg.final_ln))
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": 1.0 / dt, "unit": "windows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one full window (batch item 0) of the same workload, fp64 numpy/OpenBLAS, {dt:.1f} s",
            "cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0))}


# MI355X fp32 vector arithmetic: 256 CUs x 4 SIMDs x 32 lanes x 2 FLOP (FMA)
# x 2.4 GHz, the published 157.3 TFLOP/s.  No kernel here uses the packed-fp32
# instructions, but a SIMD issues a plain wave64 FMA in about two clocks, so
# that is the peak the log-mel kernel's arithmetic is measured against.
PEAK_F32_VALU_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12  # 157.3
# fp32 operations of one frame's STFT power in the log-mel kernel (an FMA is
# two, an add or multiply one; products by 0 and +-1 are not issued): the
# window, 400; the first stage, 20 columns x 434 (the paired real 20-point
# DFT and the twiddles); the second stage with the power, 20 rows x 673.
# The mel sums (at most 804 more: a bin lies in at most two triangles) are
# left out.
FFT_FLOPS_PER_FRAME = 400 + 20 * 434 + 20 * 673


def device_peak():
    """Dense fp16 MFMA peak from the device's own properties: CUs x 4096
    FLOP per clock (4 SIMDs x 1024) x the maximum engine clock."""
    import ctypes
    import torch
    pr = torch.cuda.get_device_properties(0)
    cus = pr.multi_processor_count
    clk = 0
    try:  # hipDeviceGetAttribute(&v, hipDeviceAttributeClockRate (5), device 0): peak clock in kHz
        hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:
            clk = v.value
    except OSError:
        pass
    out = {"name": pr.name, "gcn_arch": getattr(pr, "gcnArchName", ""), "compute_units": cus,
           "assumed_peak_tflops": PEAK_F16_TFLOPS}
    if clk:
        out["max_clock_mhz"] = clk / 1e3
        out["peak_from_clock_tflops"] = cus * 4096 * clk * 1e3 / 1e12
    return out


def time_graph(enc, mel_d, out, n_ctx, steps):
    """The same step through the library's record-once / replay entry point
    (wenc_forward_graph: the forward recorded into a hipGraph on the first
    call, launched as one graph afterwards): what a caller that replays the
    forward pays, launch overhead excluded."""
    import torch
    enc.forward_graph(mel_d, out, n_ctx=n_ctx)  # records
    enc.forward_graph(mel_d, out, n_ctx=n_ctx)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        enc.forward_graph(mel_d, out, n_ctx=n_ctx)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # per replay (median, minimum), like the eager per-call figures
    per = []
    for _ in range(max(steps // 2, 3)):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        enc.forward_graph(mel_d, out, n_ctx=n_ctx)
        c1.record(stream)
        per.append((c0, c1))
    torch.cuda.synchronize()
    call_ms = sorted(c0.elapsed_time(c1) for c0, c1 in per)
    return {"ms_per_step": ms, "value": mel_d.shape[0] / (ms * 1e-3),
            "per_call_ms": {"median": call_ms[len(call_ms) // 2], "min": call_ms[0], "calls": len(call_ms)}}


def time_frontend(enc, model, B, steps):
    """wenc_log_mel over B synthetic windows, timed with events on the stream."""
    import torch
    from whisper_audio_encoder_amd import synth, wenc
    audio = torch.from_numpy(synth.make_audio(B, n_samples=160 * model.n_frames, seed=model.seed)).to("cuda:0")
    mel = torch.empty((B, model.n_frames, model.n_mels), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        enc.log_mel(audio, mel)
    wenc.wenc_profile(enc.h, 1 << wenc.SITES.index("mel"))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        enc.log_mel(audio, mel)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    wenc.wenc_profile(enc.h, 0)
    flops = float(B * model.n_frames * FFT_FLOPS_PER_FRAME)
    tf = flops / ms / 1e9
    log(f"[bench] log-mel, {B} windows: {ms:.3f} ms per call, {tf:.1f} TFLOP/s "
        f"(the FFT's fp32 vector arithmetic, {FFT_FLOPS_PER_FRAME} per frame)")
    return {"windows": B, "ms_per_call": ms, "windows_per_s": B / (ms * 1e-3),
            "roofline": {"bound": "alu", "achieved": tf, "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / PEAK_F32_VALU_TFLOPS}}


def time_cross(enc, model, memory, n_dec, steps):
    """The decoder's cross-attention K/V of n_dec layers from the encoder
    output, timed like the forward (events on the stream, after a warm-up)."""
    import torch
    from whisper_audio_encoder_amd import synth, wenc
    enc.load_cross(synth.pack_cross_blob(model, synth.make_cross_params(model, n_dec), n_dec), n_dec)
    B, T, d = memory.shape
    xk = torch.empty((n_dec, B, T, d), dtype=torch.float16, device=memory.device)
    xv = torch.empty_like(xk)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        wenc.wenc_prepare_cross(enc.h, memory, B, T, xk, xv)
    wenc.wenc_profile(enc.h, 1 << wenc.SITES.index("xkv"))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        wenc.wenc_prepare_cross(enc.h, memory, B, T, xk, xv)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kv_ms, kv_n = wenc.wenc_profile_read(enc.h)["xkv"]
    wenc.wenc_profile(enc.h, 0)
    flops = 2.0 * B * T * 2 * d * d * n_dec
    log(f"[bench] cross K/V, {n_dec} decoder layers: {ms:.3f} ms per call, {flops / ms / 1e9:.1f} TFLOP/s")
    # one decode step's cross-attention: a query row per window over every
    # layer's cached K/V (HBM-bound: K and V read once)
    q = (torch.randn((B, 1, d), device=memory.device) * 0.5).half()
    o = torch.empty_like(q)
    for layer in range(n_dec):
        enc.cross_attend(q, xk[layer], xv[layer], out=o)
    wenc.wenc_profile(enc.h, 1 << wenc.SITES.index("xatt"))
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        for layer in range(n_dec):
            enc.cross_attend(q, xk[layer], xv[layer], out=o)
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    at_ms, at_n = wenc.wenc_profile_read(enc.h)["xatt"]
    wenc.wenc_profile(enc.h, 0)
    per_layer = at_ms / max(at_n, 1)
    kv_bytes = 2.0 * B * T * d * 2  # K and V, fp16, one layer
    log(f"[bench] decode-step cross-attention, {n_dec} layers: {step_ms:.3f} ms per step, "
        f"{per_layer * 1e3:.1f} us per layer ({kv_bytes / (per_layer * 1e-3) / 1e9:.0f} GB/s of K/V)")
    # the step's greedy token choice: argmax over N_VOCAB fp32 logits per window
    logits = torch.randn((B, N_VOCAB), device=memory.device)
    tok = enc.argmax(logits)
    wenc.wenc_profile(enc.h, 1 << wenc.SITES.index("amax"))
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        enc.argmax(logits, out=tok)
    e1.record(stream)
    torch.cuda.synchronize()
    am_call_ms = e0.elapsed_time(e1) / steps
    am_ms, am_n = wenc.wenc_profile_read(enc.h)["amax"]
    wenc.wenc_profile(enc.h, 0)
    am_launch = am_ms / max(am_n, 1)
    am_bytes = B * N_VOCAB * 4.0
    log(f"[bench] decode-step argmax over {N_VOCAB} logits x {B} rows: {am_launch * 1e3:.1f} us per call "
        f"({am_bytes / (am_launch * 1e-3) / 1e9:.0f} GB/s)")
    return {"n_dec_layer": n_dec, "ms_per_call": ms, "tflops": flops / ms / 1e9,
            "gemm_avg_launch_ms": kv_ms / max(kv_n, 1),
            "decode_step_attention": {"n_q": 1, "ms_per_step": step_ms, "us_per_layer": per_layer * 1e3,
                                      "kv_gb_per_s": kv_bytes / (per_layer * 1e-3) / 1e9,
                                      "roofline": {"bound": "hbm", "achieved": kv_bytes / (per_layer * 1e-3) / 1e9,
                                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                                   "frac": kv_bytes / (per_layer * 1e-3) / 1e9 / PEAK_HBM_GBS}},
            "decode_step_argmax": {"rows": B, "n_vocab": N_VOCAB, "us_per_call": am_launch * 1e3,
                                   "us_per_call_stream": am_call_ms * 1e3,
                                   "gb_per_s": am_bytes / (am_launch * 1e-3) / 1e9}}


def site_launches_per_step(cfg, site):
    """How many times a site runs over the whole batch in one step."""
    return cfg.n_layer if site in ("ln1", "qkv", "attn", "oproj", "ln2", "fc1", "fc2") else 1


def run_workload(name, a, with_cpu):
    """Time `steps` forwards of one workload's batch (after `warmup`) and
    return its measurements: throughput, the dominant kernel's roofline
    from events over the timed region, per-call and hipGraph figures, and
    the oracle's CPU baseline."""
    import torch
    from whisper_audio_encoder_amd import synth, wenc
    from whisper_audio_encoder_amd.configs import CONFIGS, WORKLOAD_NAMES

    model = CONFIGS[name]
    B = a.batch or model.batch
    # cfg: the shape each window is encoded at (a draft runs the same model over fewer positions)
    cfg = model if a.n_ctx is None else model.with_(n_ctx=a.n_ctx, n_frames=2 * a.n_ctx)
    log(f"[bench] workload {name}: {WORKLOAD_NAMES[name]}; running batch {B}"
        + ("" if a.n_ctx is None else f", drafts of {a.n_ctx} positions"))
    mel, params = synth.make_inputs(model, batch=B)
    mel = np.ascontiguousarray(mel[:, :cfg.n_frames])
    blob = synth.pack_blob(model, params)
    enc = wenc.Encoder(model, blob, max_batch=B)
    mel_d = torch.from_numpy(mel).to("cuda:0")
    out = torch.empty((B, cfg.n_ctx, cfg.d_model), dtype=torch.float32, device="cuda:0")
    n_ctx = a.n_ctx
    stream = torch.cuda.current_stream()

    def timed(e, steps):
        """ms per forward over `steps` forwards, events on the caller's stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            e.forward(mel_d, out, n_ctx=n_ctx)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # warm-up (the first forward loads the code objects), then the timed
    # region: the forward as a caller runs it, no events inside
    for _ in range(max(a.warmup, 1)):
        enc.forward(mel_d, out, n_ctx=n_ctx)
    t0 = time.perf_counter()
    ms = timed(enc, a.steps)
    wall = time.perf_counter() - t0
    log(f"[bench] {name}: {a.steps} steps: {ms:.3f} ms/step (wall {1e3 * wall / a.steps:.3f} ms/step)")
    # per-call times (median, minimum) from events around each forward
    per_call = []
    for _ in range(max(a.steps // 2, 3)):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        enc.forward(mel_d, out, n_ctx=n_ctx)
        c1.record(stream)
        per_call.append((c0, c1))
    torch.cuda.synchronize()
    call_ms = sorted(c0.elapsed_time(c1) for c0, c1 in per_call)
    graph = time_graph(enc, mel_d, out, n_ctx, a.steps)
    log(f"[bench] {name}: hipGraph replay: {graph['ms_per_step']:.3f} ms/step")

    # The kernels' own rates.  The forward above splits its windows over two
    # streams, so kernels of different sites overlap and no launch's time
    # is its own.  A second handle runs the same forward with every launch on
    # the caller's stream (WENC_SPLIT_STREAMS=1): its warm-up, with events
    # around every launch, finds the dominant site; its timed steps, with
    # events around that site's launches only, give the roofline.
    saved = os.environ.get("WENC_SPLIT_STREAMS")
    os.environ["WENC_SPLIT_STREAMS"] = "1"
    try:
        enc1 = wenc.Encoder(model, blob, max_batch=B)
    finally:
        if saved is None:
            del os.environ["WENC_SPLIT_STREAMS"]
        else:
            os.environ["WENC_SPLIT_STREAMS"] = saved
    enc1.forward(mel_d, out, n_ctx=n_ctx)
    n_warm = max(a.warmup - 1, 1)
    wenc.wenc_profile(enc1.h, (1 << wenc.N_SITES) - 1)
    timed(enc1, n_warm)
    warm = wenc.wenc_profile_read(enc1.h)
    dominant = max(wenc.SITES, key=lambda s: warm[s][0])
    total_warm = sum(v[0] for v in warm.values()) or 1.0
    log("[bench] per-site share of kernel time (one stream, warm-up): " +
        ", ".join(f"{s} {100 * warm[s][0] / total_warm:.1f}%" for s in wenc.SITES if warm[s][1]))
    wenc.wenc_profile(enc1.h, 1 << wenc.SITES.index(dominant))
    ms1 = timed(enc1, a.steps)
    prof = wenc.wenc_profile_read(enc1.h)
    wenc.wenc_profile(enc1.h, 0)
    enc1.close()
    log(f"[bench] {name}: one stream: {ms1:.3f} ms/step")

    flops = cfg.flops_per_window() * B
    tflops = flops / (ms * 1e-3) / 1e12
    # The dominant site over the whole batch, on one stream: its algorithmic
    # work per application (all windows) over its time per application (the
    # library's events bracket each launch; a site launched as two kernels,
    # fc1's two tile sizes, counts both).
    kind, work = site_work(cfg, B)[dominant]
    d_ms, d_n = prof[dominant]
    per_step = site_launches_per_step(cfg, dominant)
    avg_s = d_ms / (a.steps * per_step) * 1e-3
    if kind == "mfma":
        roof = {"bound": "mfma", "achieved": work / avg_s / 1e12, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": work / avg_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(name, dominant)
    roof["kernel"] = dominant
    roof["avg_launch_ms"] = avg_s * 1e3
    roof["launches"] = d_n
    roof["applications"] = a.steps * per_step
    roof["measured_on"] = ("one stream: the timed steps of a second handle whose forward keeps every launch "
                           "on the caller's stream")

    frontend = time_frontend(enc, model, B, a.steps) if a.frontend else None
    cross = time_cross(enc, model, out, a.cross, a.steps) if a.cross else None

    cpu = None
    if with_cpu:
        log(f"[bench] {name}: timing the fp64 oracle on one window ...")
        cpu = cpu_baseline(cfg, mel, params)
        log(f"[bench] oracle: {cpu['value']:.4f} windows/s on {cpu['cores']} threads")

    rec = {
        "value": B / (ms * 1e-3),
        "unit": "windows/s",
        "ms_per_step": ms,
        "config": {"workload": f"{WORKLOAD_NAMES[name]} ({name})"
                   + ("" if n_ctx is None else f", drafts: {cfg.n_frames} frames per window"), "batch": B,
                   "n_frames": cfg.n_frames, "n_ctx": cfg.n_ctx, "d_model": cfg.d_model, "n_head": cfg.n_head,
                   "d_ff": cfg.d_ff, "n_layer": cfg.n_layer, "n_mels": cfg.n_mels, "parallelism": "single GPU"},
        "tflops": tflops,
        "pct_fp16_peak": 100.0 * tflops / PEAK_F16_TFLOPS,
        "per_call_ms": {"median": call_ms[len(call_ms) // 2], "min": call_ms[0], "calls": len(call_ms)},
        "graph_replay": graph,
        "one_stream": {"ms_per_step": ms1, "value": B / (ms1 * 1e-3)},
        "site_ms_per_step": {s: warm[s][0] / n_warm for s in wenc.SITES if warm[s][1]},
        "roofline": roof,
        "cpu_baseline": cpu,
        **({"cross_kv": cross} if cross else {}),
        **({"log_mel": frontend} if frontend else {}),
    }
    enc.close()
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=["c0", "c1", "c2", "c3", "c4"])
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured after the headline one, each reported as a nested "
                         "record under its name (default: c3 when the headline is c4, the other config the "
                         "50%%-of-peak target names; '' for none)")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch")
    ap.add_argument("--n-ctx", type=int, default=None,
                    help="shortened context (drafts): encode 2*N_CTX frames per window with the full model")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--frontend", action="store_true",
                    help="also time the log-mel frontend on the same number of synthetic 30-s windows")
    ap.add_argument("--cross", type=int, default=None, metavar="N_DEC",
                    help="also time the cross-attention K/V projection of N_DEC decoder layers from the output")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration) and exit")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only time the LayerNorm against torch conversions moving the same bytes and exit")
    ap.add_argument("--gemm-tile-costs", action="store_true",
                    help="only measure the 256 x 256 GEMM's cost per k step and per tile and exit")
    a = ap.parse_args(argv)
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    if a.gemm_tile_costs:
        gemm_tile_costs()
        return
    if a.hbm_ceiling:
        hbm_ceiling()
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the encoder shards by window (pure data parallelism, no "
              "collective), and this build runs and reports a single MI355X only", file=sys.stderr)
        sys.exit(2)
    also = a.also
    if also is None:
        also = "c3" if a.workload == "c4" and a.batch is None and a.n_ctx is None else ""
    also = [w for w in also.split(",") if w and w != a.workload]

    head = run_workload(a.workload, a, not a.no_cpu_baseline)
    nested = {}
    for w in also:
        sub = argparse.Namespace(**{**vars(a), "frontend": False, "cross": None})
        rec = run_workload(w, sub, not a.no_cpu_baseline)
        nested[w] = {"metric": METRIC, "steps": a.steps, "warmup": a.warmup, **rec}

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "windows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded mel N(-0.2,0.4) clamped, random-init fp16 weights)",
        **{k: v for k, v in head.items() if k not in ("value", "unit", "ms_per_step")},
        "device_peak": device_peak(),
        **nested,
        "host": platform.node(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
