"""ctypes binding of libwenc.so (C ABI in include/wenc.h).

Argument marshalling only: every step of the encoder runs in the library's
HIP kernels.  Device buffers are torch tensors (``.data_ptr()``) and the
stream is torch's current HIP stream unless one is given.  The functions
carry the C names; ``Encoder`` bundles create + load + forward.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (both are ``libamdhip64.so.7``), which
makes torch's stream handles and device pointers valid inside it.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

from .configs import EncoderConfig

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwenc.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "wenc.h")

WENC_OK, WENC_EINVAL, WENC_ENOMEM, WENC_ENODEV, WENC_ESTATE, WENC_EHIP = 0, -1, -2, -3, -4, -5
WENC_TAP_C1, WENC_TAP_STEM, WENC_TAP_BLOCK = 0, 1, 2
WENC_EPI_GELU_F16, WENC_EPI_CONV2, WENC_EPI_RESID, WENC_EPI_QKV, WENC_EPI_KV = 0, 1, 2, 3, 4
SITES = ("ingest", "conv1", "conv2", "ln1", "qkv", "attn", "oproj", "ln2", "fc1", "fc2", "lnf", "xcvt", "xkv", "mel", "xatt", "amax")
N_SITES = len(SITES)


class WencError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"wenc error {code}: {msg}")
        self.code = code


class wenc_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_mels", "d_model", "n_head", "head_dim", "d_ff", "n_layer",
                                              "n_frames", "n_ctx")] + \
               [("ln_eps", ctypes.c_float), ("final_ln", ctypes.c_int32), ("max_batch", ctypes.c_int32)]


class wenc_gemm_args(ctypes.Structure):
    _fields_ = [
        ("A", ctypes.c_void_p), ("a_batch_stride", ctypes.c_int64), ("a_rows_per_batch", ctypes.c_int32),
        ("lda", ctypes.c_int32),
        ("W", ctypes.c_void_p), ("ldw", ctypes.c_int32),
        ("bias", ctypes.c_void_p),
        ("C", ctypes.c_void_p), ("c_batch_stride", ctypes.c_int64), ("c_rows_per_batch", ctypes.c_int32),
        ("c_row_offset", ctypes.c_int32), ("ldc", ctypes.c_int32),
        ("pos", ctypes.c_void_p), ("pos_rows", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("vt", ctypes.c_void_p), ("T", ctypes.c_int32),
        ("n_head", ctypes.c_int32), ("ldvt", ctypes.c_int32), ("q_scale", ctypes.c_float),
        ("M", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("epilogue", ctypes.c_int32),
        ("C2", ctypes.c_void_p), ("n_split", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libwenc.so (once).  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m whisper_audio_encoder_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(wenc_config)
    L.wenc_create.argtypes = [cfgp, ctypes.POINTER(vp)]
    L.wenc_create.restype = ctypes.c_int
    L.wenc_weights_nbytes.argtypes = [cfgp]
    L.wenc_weights_nbytes.restype = sz
    L.wenc_load.argtypes = [vp, vp, sz]
    L.wenc_load.restype = ctypes.c_int
    L.wenc_forward.argtypes = [vp, vp, i32, vp, vp]
    L.wenc_forward.restype = ctypes.c_int
    L.wenc_cross_nbytes.argtypes = [cfgp, i32]
    L.wenc_cross_nbytes.restype = sz
    L.wenc_load_cross.argtypes = [vp, i32, vp, sz]
    L.wenc_load_cross.restype = ctypes.c_int
    L.wenc_prepare_cross.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    L.wenc_cross_attend.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp]
    L.wenc_cross_attend.restype = ctypes.c_int
    L.wenc_k_gemm_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(i32)]
    L.wenc_k_gemm_plan.restype = ctypes.c_int
    L.wenc_k_logmel_tables.argtypes = [i32, ctypes.POINTER(i32), vp, vp, ctypes.c_int64]
    L.wenc_k_logmel_tables.restype = ctypes.c_int
    L.wenc_argmax.argtypes = [vp, vp, i32, i32, ctypes.c_int64, vp, vp]
    L.wenc_argmax.restype = ctypes.c_int
    L.wenc_argmax_noalloc.argtypes = [vp, i32, i32, ctypes.c_int64, vp, vp]
    L.wenc_argmax_noalloc.restype = ctypes.c_int
    L.wenc_prepare_cross.restype = ctypes.c_int
    L.wenc_log_mel.argtypes = [vp, vp, i32, vp, vp]
    L.wenc_log_mel.restype = ctypes.c_int
    L.wenc_forward_ctx.argtypes = [vp, vp, i32, i32, vp, vp]
    L.wenc_forward_ctx.restype = ctypes.c_int
    L.wenc_forward_graph.argtypes = [vp, vp, i32, i32, vp, vp]
    L.wenc_forward_graph.restype = ctypes.c_int
    L.wenc_forward_tap.argtypes = [vp, vp, i32, i32, vp, vp]
    L.wenc_forward_tap.restype = ctypes.c_int
    L.wenc_destroy.argtypes = [vp]
    L.wenc_destroy.restype = None
    L.wenc_last_error.argtypes = [vp]
    L.wenc_last_error.restype = ctypes.c_char_p
    L.wenc_k_layernorm.argtypes = [vp, vp, vp, vp, i32, i32, ctypes.c_float, i32, vp]
    L.wenc_k_layernorm.restype = ctypes.c_int
    L.wenc_k_gemm.argtypes = [ctypes.POINTER(wenc_gemm_args), vp]
    L.wenc_k_gemm.restype = ctypes.c_int
    L.wenc_k_gemm_mode.argtypes = [i32, i32]
    L.wenc_k_gemm_mode.restype = ctypes.c_int
    L.wenc_k_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp]
    L.wenc_k_attention.restype = ctypes.c_int
    L.wenc_profile.argtypes = [vp, ctypes.c_uint32]
    L.wenc_profile.restype = ctypes.c_int
    L.wenc_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.wenc_profile_read.restype = ctypes.c_int
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/wenc.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wenc_[a-z_0-9]+)\s*\(", src)))


def _check(rc: int, h=None):
    if rc != WENC_OK:
        raise WencError(rc, wenc_last_error(h))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def make_config(cfg: EncoderConfig, max_batch: int | None = None) -> wenc_config:
    return wenc_config(cfg.n_mels, cfg.d_model, cfg.n_head, cfg.head_dim, cfg.d_ff, cfg.n_layer,
                       cfg.n_frames, cfg.n_ctx, cfg.ln_eps, cfg.final_ln,
                       cfg.batch if max_batch is None else max_batch)


# ---------------------------------------------------------------- C names
def wenc_last_error(h=None) -> str:
    return lib().wenc_last_error(h).decode()


def wenc_weights_nbytes(cfg: wenc_config) -> int:
    return lib().wenc_weights_nbytes(ctypes.byref(cfg))


def wenc_create(cfg: wenc_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib().wenc_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def wenc_load(h, blob: np.ndarray) -> None:
    blob = np.ascontiguousarray(blob).view(np.uint8)
    _check(lib().wenc_load(h, blob.ctypes.data, blob.nbytes), h)


def wenc_forward(h, mel: torch.Tensor, batch: int, out: torch.Tensor, stream=None) -> None:
    _check(lib().wenc_forward(h, _ptr(mel), batch, _ptr(out), _stream(stream)), h)


def wenc_forward_ctx(h, mel: torch.Tensor, batch: int, n_ctx: int, out: torch.Tensor, stream=None) -> None:
    _check(lib().wenc_forward_ctx(h, _ptr(mel), batch, n_ctx, _ptr(out), _stream(stream)), h)


def wenc_forward_graph(h, mel: torch.Tensor, batch: int, n_ctx: int, out: torch.Tensor, stream=None) -> None:
    _check(lib().wenc_forward_graph(h, _ptr(mel), batch, n_ctx, _ptr(out), _stream(stream)), h)


def wenc_log_mel(h, audio: torch.Tensor, batch: int, mel: torch.Tensor, stream=None) -> None:
    _check(lib().wenc_log_mel(h, _ptr(audio), batch, _ptr(mel), _stream(stream)), h)


def wenc_cross_nbytes(cfg: wenc_config, n_dec_layer: int) -> int:
    return lib().wenc_cross_nbytes(ctypes.byref(cfg), n_dec_layer)


def wenc_load_cross(h, n_dec_layer: int, blob: np.ndarray) -> None:
    blob = np.ascontiguousarray(blob)
    _check(lib().wenc_load_cross(h, n_dec_layer, blob.ctypes.data, blob.nbytes), h)


def wenc_prepare_cross(h, memory: torch.Tensor, batch: int, n_ctx: int, xk: torch.Tensor, xv: torch.Tensor,
                       stream=None) -> None:
    _check(lib().wenc_prepare_cross(h, _ptr(memory), batch, n_ctx, _ptr(xk), _ptr(xv), _stream(stream)), h)


def wenc_cross_attend(h, q: torch.Tensor, xk: torch.Tensor, xv: torch.Tensor, batch: int, n_q: int, n_ctx: int,
                      out: torch.Tensor, stream=None) -> None:
    _check(lib().wenc_cross_attend(h, _ptr(q), _ptr(xk), _ptr(xv), batch, n_q, n_ctx, _ptr(out), _stream(stream)), h)


def wenc_k_logmel_tables(n_mels: int):
    """Host-side mel-filter tables of wenc_log_mel: (mstart [n_mels] int32,
    mwt [n_mels][16 nch] fp32), see wenc.h."""
    import numpy as np
    nch = ctypes.c_int32()
    if lib().wenc_k_logmel_tables(n_mels, ctypes.byref(nch), None, None, 0) != WENC_OK:
        raise ValueError(f"wenc_k_logmel_tables: {wenc_last_error()}")
    mstart = np.zeros(n_mels, dtype=np.int32)
    mwt = np.zeros((n_mels, 16 * nch.value), dtype=np.float32)
    rc = lib().wenc_k_logmel_tables(n_mels, ctypes.byref(nch), mstart.ctypes.data, mwt.ctypes.data, mwt.size)
    if rc != WENC_OK:
        raise ValueError(f"wenc_k_logmel_tables: {wenc_last_error()}")
    return mstart, mwt


def wenc_k_gemm_plan(M: int, N: int, cus: int = 256, tile: int = -1, split: int = 1,
                     streams: int = 1) -> tuple[int, int]:
    """Host-side tile plan of a GEMM launch: (kind, big_rows), see wenc.h."""
    rows = ctypes.c_int32()
    kind = lib().wenc_k_gemm_plan(M, N, cus, tile, split, streams, ctypes.byref(rows))
    if kind < 0:
        raise ValueError(f"wenc_k_gemm_plan: {wenc_last_error()}")
    return kind, rows.value


def wenc_argmax(h, logits: torch.Tensor, rows: int, n_vocab: int, ld: int, out: torch.Tensor, stream=None) -> None:
    _check(lib().wenc_argmax(h, _ptr(logits), rows, n_vocab, ld, _ptr(out), _stream(stream)), h)


def wenc_argmax_noalloc(logits: torch.Tensor, rows: int, n_vocab: int, ld: int, out: torch.Tensor,
                        stream=None) -> None:
    _check(lib().wenc_argmax_noalloc(_ptr(logits), rows, n_vocab, ld, _ptr(out), _stream(stream)))


def wenc_forward_tap(h, mel: torch.Tensor, batch: int, tap: int, dst: torch.Tensor, stream=None) -> None:
    _check(lib().wenc_forward_tap(h, _ptr(mel), batch, tap, _ptr(dst), _stream(stream)), h)


def wenc_destroy(h) -> None:
    lib().wenc_destroy(h)


def wenc_k_layernorm(x, gamma, beta, y, rows, d, eps, out_f32, stream=None) -> None:
    _check(lib().wenc_k_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, d, eps, int(out_f32),
                                  _stream(stream)))


def wenc_k_gemm(args: wenc_gemm_args, stream=None) -> None:
    _check(lib().wenc_k_gemm(ctypes.byref(args), _stream(stream)))


def wenc_k_attention(q, k, vt, ao, batch, n_head, T, ldvt, stream=None) -> None:
    _check(lib().wenc_k_attention(_ptr(q), _ptr(k), _ptr(vt), _ptr(ao), batch, n_head, T, ldvt, _stream(stream)))


def wenc_profile(h, site_mask: int) -> None:
    _check(lib().wenc_profile(h, site_mask), h)


def wenc_profile_read(h) -> dict:
    ms = (ctypes.c_double * N_SITES)()
    n = (ctypes.c_int64 * N_SITES)()
    _check(lib().wenc_profile_read(h, ms, n), h)
    return {SITES[i]: (ms[i], n[i]) for i in range(N_SITES)}


# ---------------------------------------------------------------- wrapper
class Encoder:
    """One loaded encoder on the current device."""

    def __init__(self, cfg: EncoderConfig, blob: np.ndarray, max_batch: int | None = None):
        self.cfg = cfg
        self.ccfg = make_config(cfg, max_batch)
        self.h = wenc_create(self.ccfg)
        try:
            wenc_load(self.h, blob)
        except Exception:
            wenc_destroy(self.h)
            self.h = None
            raise

    def _check_mel(self, mel: torch.Tensor, n_frames: int | None = None):
        c = self.cfg
        n_frames = c.n_frames if n_frames is None else n_frames
        if not (mel.is_cuda and mel.dtype == torch.float32 and mel.is_contiguous()):
            raise ValueError("mel must be a contiguous fp32 device tensor")
        if mel.dim() != 3 or mel.shape[1:] != (n_frames, c.n_mels):
            raise ValueError(f"mel must be [batch, {n_frames}, {c.n_mels}], got {tuple(mel.shape)}")

    def forward(self, mel: torch.Tensor, out: torch.Tensor | None = None, stream=None,
                n_ctx: int | None = None) -> torch.Tensor:
        """Encode full windows, or with ``n_ctx`` a shortened context (drafts):
        mel [batch, 2 n_ctx, n_mels] -> out [batch, n_ctx, d_model]."""
        c = self.cfg
        T = c.n_ctx if n_ctx is None else n_ctx
        self._check_mel(mel, 2 * T)
        B = mel.shape[0]
        if out is None:
            out = torch.empty((B, T, c.d_model), dtype=torch.float32, device=mel.device)
        elif not (out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()
                  and tuple(out.shape) == (B, T, c.d_model)):
            raise ValueError(f"out must be a contiguous fp32 device tensor [batch, {T}, d_model]")
        if n_ctx is None:
            wenc_forward(self.h, mel, B, out, stream)
        else:
            wenc_forward_ctx(self.h, mel, B, n_ctx, out, stream)
        return out

    def forward_graph(self, mel: torch.Tensor, out: torch.Tensor | None = None, stream=None,
                      n_ctx: int | None = None) -> torch.Tensor:
        """forward() through the library's recorded graph: recorded on the
        first call for these buffers and sizes, replayed afterwards."""
        c = self.cfg
        T = c.n_ctx if n_ctx is None else n_ctx
        self._check_mel(mel, 2 * T)
        B = mel.shape[0]
        if out is None:
            out = torch.empty((B, T, c.d_model), dtype=torch.float32, device=mel.device)
        elif not (out.is_cuda and out.dtype == torch.float32 and out.is_contiguous()
                  and tuple(out.shape) == (B, T, c.d_model)):
            raise ValueError(f"out must be a contiguous fp32 device tensor [batch, {T}, d_model]")
        wenc_forward_graph(self.h, mel, B, T, out, stream)
        return out

    def log_mel(self, audio: torch.Tensor, mel: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Log-mel of whole windows: audio [batch, 160 n_frames] fp32 ->
        mel [batch, n_frames, n_mels] fp32, the layout forward() reads."""
        c = self.cfg
        if not (audio.is_cuda and audio.dtype == torch.float32 and audio.is_contiguous()
                and audio.dim() == 2 and audio.shape[1] == 160 * c.n_frames):
            raise ValueError(f"audio must be a contiguous fp32 device tensor [batch, {160 * c.n_frames}]")
        B = audio.shape[0]
        if mel is None:
            mel = torch.empty((B, c.n_frames, c.n_mels), dtype=torch.float32, device=audio.device)
        wenc_log_mel(self.h, audio, B, mel, stream)
        return mel

    def load_cross(self, blob: np.ndarray, n_dec_layer: int) -> None:
        """Load the decoder layers' cross-attention K/V weights (x_wk, x_wv, x_bv)."""
        wenc_load_cross(self.h, n_dec_layer, blob)
        self.n_dec_layer = n_dec_layer

    def prepare_cross(self, memory: torch.Tensor, stream=None):
        """Cross-attention K and V of every loaded decoder layer from the
        encoder memory [batch, n_ctx, d_model] fp32: two fp16 tensors
        [n_dec_layer, batch, n_ctx, d_model]."""
        c = self.cfg
        if not (memory.is_cuda and memory.dtype == torch.float32 and memory.is_contiguous()
                and memory.dim() == 3 and memory.shape[2] == c.d_model):
            raise ValueError("memory must be a contiguous fp32 device tensor [batch, n_ctx, d_model]")
        B, T = memory.shape[0], memory.shape[1]
        n = getattr(self, "n_dec_layer", 0)
        xk = torch.empty((n, B, T, c.d_model), dtype=torch.float16, device=memory.device)
        xv = torch.empty_like(xk)
        wenc_prepare_cross(self.h, memory, B, T, xk, xv, stream)
        return xk, xv

    def cross_attend(self, q: torch.Tensor, xk: torch.Tensor, xv: torch.Tensor, out=None, stream=None):
        """Decode-step cross-attention of q [batch, n_q, d_model] fp16 over
        one decoder layer's xk, xv [batch, n_ctx, d_model] fp16 (a slice of
        prepare_cross's output): fp16 [batch, n_q, d_model]."""
        c = self.cfg
        for name, t in (("q", q), ("xk", xk), ("xv", xv)):
            if not (t.is_cuda and t.dtype == torch.float16 and t.is_contiguous() and t.dim() == 3
                    and t.shape[2] == c.d_model):
                raise ValueError(f"{name} must be a contiguous fp16 device tensor [batch, rows, d_model]")
        if xk.shape != xv.shape or xk.shape[0] != q.shape[0]:
            raise ValueError("xk and xv must match, with q's batch")
        if out is None:
            out = torch.empty_like(q)
        wenc_cross_attend(self.h, q, xk, xv, q.shape[0], q.shape[1], xk.shape[1], out, stream)
        return out

    def argmax(self, logits: torch.Tensor, out=None, stream=None) -> torch.Tensor:
        """Greedy token choice: per row of logits [rows, n_vocab] fp32 (rows
        may be strided), the index of the largest value: int32 [rows]."""
        if not (logits.is_cuda and logits.dtype == torch.float32 and logits.dim() == 2
                and logits.stride(1) == 1 and logits.stride(0) >= logits.shape[1]):
            raise ValueError("logits must be an fp32 device tensor [rows, n_vocab] with unit column stride")
        rows, n = logits.shape
        if out is None:
            out = torch.empty((rows,), dtype=torch.int32, device=logits.device)
        elif not (out.is_cuda and out.dtype == torch.int32 and out.is_contiguous() and out.shape == (rows,)):
            raise ValueError("out must be a contiguous int32 device tensor [rows]")
        wenc_argmax(self.h, logits, rows, n, logits.stride(0), out, stream)
        return out

    def tap(self, mel: torch.Tensor, tap: int, stream=None) -> torch.Tensor:
        self._check_mel(mel)
        c = self.cfg
        B = mel.shape[0]
        if tap == WENC_TAP_C1:
            dst = torch.empty((B, c.n_frames, c.d_model), dtype=torch.float16, device=mel.device)
        else:
            dst = torch.empty((B, c.n_ctx, c.d_model), dtype=torch.float32, device=mel.device)
        wenc_forward_tap(self.h, mel, B, tap, dst, stream)
        return dst

    def close(self):
        if self.h is not None:
            wenc_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
