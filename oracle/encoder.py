"""Plain fp64 definition of the Whisper audio-encoder forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import or call this module.

Every function evaluates the operation's definition in float64 with numpy,
using a matrix product or scipy's erf as a library step and nothing else:
no blocking, no fusion, no online softmax, no reduced precision.  Inputs are
the exact values the GPU consumes (fp16 parameters and fp32 mel widened to
fp64 without rounding).

Sources (the pages the method is described on):

* whisper 0.9.0 API page, section model.nu: conv1 (k=3, s=1, pad=1) then
  GELU, conv2 (k=3, s=2, pad=1) then GELU, 3000 -> 1500 frames; a stored
  position table; N x [LN -> non-causal self-attention -> +residual,
  LN -> fc1 -> GELU -> fc2 -> +residual], then LN; k_proj has no bias.
* same page, section kernels.nu: LayerNorm subtracts the mean and has a bias;
  GELU is the error-function form, not the tanh approximation; attention is
  non-causal; scores are q.k / sqrt(head_dim).
* CKE page ("How Audio Becomes Words"), sections "The Encoder: Understand
  Once" (full 1500 x 1500 square, no mask, no RoPE) and the stitched-circuit
  figure (conv1d s1, gelu, conv1d s2, gelu, + positions; LN, q/k/v proj,
  attention, out_proj, residual; LN, d -> 4d, gelu, 4d -> d, residual;
  final_norm).

Readings where the pages are silent (all recorded in the design notes):
cross-correlation without kernel flip, conv taps stored [out][in][k], zero
padding of one frame each side, population variance with eps inside the
square root, GELU(z) = z/2 * (1 + erf(z / sqrt 2)), head h owns columns
[64h, 64h+64), a zero bias for k.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


def conv1d(x, w, b, stride: int, pad: int = 1) -> np.ndarray:
    """One 1-D convolution layer of the stem (model.nu: k=3, pad=1, s=1 or 2).

    x: [T_in, C_in] frame-contiguous (whisper 0.9.0 API page, wh_encode: a
    frame is contiguous).  w: [C_out, C_in, K].  b: [C_out].
    y[t, o] = b[o] + sum_j sum_c w[o, c, j] * x[stride*t + j - pad, c], with
    x outside [0, T_in) read as zero; T_out = (T_in + 2*pad - K) // stride + 1.
    """
    x, w, b = _f64(x), _f64(w), _f64(b)
    T_in, C_in = x.shape
    C_out, C_in_w, K = w.shape
    assert C_in_w == C_in
    T_out = (T_in + 2 * pad - K) // stride + 1
    xp = np.zeros((T_in + 2 * pad, C_in), dtype=F64)
    xp[pad:pad + T_in] = x
    y = np.broadcast_to(b, (T_out, C_out)).copy()
    for j in range(K):
        # rows of the padded input that tap j reads: stride*t + j for t < T_out
        rows = xp[j: j + stride * (T_out - 1) + 1: stride]
        y += rows @ w[:, :, j].T
    return y


def gelu(z) -> np.ndarray:
    """Exact GELU, the error-function form (kernels.nu: not the tanh form)."""
    z = _f64(z)
    return 0.5 * z * (1.0 + _erf(z / np.sqrt(2.0)))


def layer_norm(x, g, b, eps: float) -> np.ndarray:
    """LayerNorm over the last axis with gain and bias (kernels.nu: it
    subtracts the mean and has a bias).  Population variance, eps inside the
    square root."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(g) + _f64(b)


def softmax_rows(s) -> np.ndarray:
    """Row softmax, shifted by the row maximum."""
    s = _f64(s)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention(q, k, v) -> np.ndarray:
    """Single-head non-causal attention: softmax(q k^T / sqrt(hd)) v.

    kernels.nu (wk_attn, causal 0: every query sees every key) and the CKE
    page (full square score grid, no mask).  The score matrix is formed in
    full, as the unfused attn_sc / attn_out pair on the API page does.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    hd = q.shape[-1]
    s = (q @ k.T) / np.sqrt(hd)
    return softmax_rows(s) @ v


def mha(xn, p: dict, n_head: int) -> np.ndarray:
    """Self-attention sublayer without the residual: out_proj(attn(q, k, v)).

    q = xn Wq^T + bq, k = xn Wk^T (k_proj has no bias, model.nu),
    v = xn Wv^T + bv; head h uses columns [hd*h, hd*(h+1)); the heads'
    outputs are concatenated in that order before out_proj (+ bo).
    """
    xn = _f64(xn)
    d = xn.shape[1]
    hd = d // n_head
    q = xn @ _f64(p["wq"]).T + _f64(p["bq"])
    k = xn @ _f64(p["wk"]).T
    v = xn @ _f64(p["wv"]).T + _f64(p["bv"])
    ao = np.empty_like(q)
    for h in range(n_head):
        c = slice(h * hd, (h + 1) * hd)
        ao[:, c] = attention(q[:, c], k[:, c], v[:, c])
    return ao @ _f64(p["wo"]).T + _f64(p["bo"])


def encoder_block(x, p: dict, n_head: int, eps: float) -> np.ndarray:
    """One pre-LN block (model.nu): x += attn(LN1 x); x += fc2(gelu(fc1(LN2 x)))."""
    x = _f64(x)
    x = x + mha(layer_norm(x, p["ln1_g"], p["ln1_b"], eps), p, n_head)
    xn = layer_norm(x, p["ln2_g"], p["ln2_b"], eps)
    hmid = gelu(xn @ _f64(p["fc1_w"]).T + _f64(p["fc1_b"]))
    return x + hmid @ _f64(p["fc2_w"]).T + _f64(p["fc2_b"])


def _layer(params: dict, li: int) -> dict:
    pre = f"l{li}."
    return {k[len(pre):]: v for k, v in params.items() if k.startswith(pre)}


def encode(mel, params: dict, n_layer: int, n_head: int, eps: float = 1e-5,
           final_ln: bool = True, taps: bool = False):
    """Encoder forward of ONE window.

    mel: [n_frames, n_mels] (3000 x n_mels for a full 30 s window).  params:
    the canonical parameter dict (conv1_w, conv1_b, conv2_w, conv2_b, pos,
    l{i}.<field>, lnf_g, lnf_b).  Returns the [n_frames // 2, d] memory in
    fp64, or with ``taps=True`` a dict holding the stage outputs ``c1``
    (after conv1+GELU), ``x0`` (after conv2+GELU+positions), ``blocks`` (x
    after each block) and ``out``.

    A shorter mel is a shortened-context window (drafts: whisper
    README, section Serving: the audio plus 5 s instead of 30 s, as
    whisper.cpp's audio_ctx).  Reading: the same layers run over T =
    n_frames // 2 positions, position t adds row t of the stored table (its
    first T rows), and attention spans those T positions.
    """
    c1 = gelu(conv1d(mel, params["conv1_w"], params["conv1_b"], stride=1))
    stem = gelu(conv1d(c1, params["conv2_w"], params["conv2_b"], stride=2))
    pos = _f64(params["pos"])
    assert stem.shape[0] <= pos.shape[0], "more positions than the stored table holds"
    x = stem + pos[:stem.shape[0]]
    x0 = x
    blocks = []
    for li in range(n_layer):
        x = encoder_block(x, _layer(params, li), n_head, eps)
        if taps:
            blocks.append(x)
    out = layer_norm(x, params["lnf_g"], params["lnf_b"], eps) if final_ln else x
    if taps:
        return {"c1": c1, "x0": x0, "blocks": blocks, "out": out}
    return out


def cross_kv(memory, x_wk, x_wv, x_bv):
    """Cross-attention keys and values of one decoder layer, projected from
    the encoder memory once per clip (whisper 0.9.0 API page, wh_prepare_cross;
    model.nu: x_wk has no bias, x_wv has x_bv; CKE page, "The Decoder": the
    memory is frozen, so its K/V are computed once and cached).

    memory: [T, d] (the encoder output).  Returns (K, V), each [T, d]:
    K = memory . x_wk^T, V = memory . x_wv^T + x_bv, in fp64.
    """
    m = _f64(memory)
    return m @ _f64(x_wk).T, m @ _f64(x_wv).T + _f64(x_bv)


def cross_attend(q, xk, xv, n_head: int) -> np.ndarray:
    """Decoder cross-attention of a decode step's query rows over the cached
    K/V of one decoder layer (whisper README, "Performance and memory": the
    one-query attention a generated token runs over the 1500 encoder
    positions; whisper 0.9.0 API page, wh_prepare_cross: xk and xv hold
    n_ctx x d_model per decoder layer; kernels.nu: scores q.k / sqrt(hd)).

    q: [n_q, d] (the step's query rows, after q_proj); xk, xv: [T, d].  Head
    h uses columns [hd*h, hd*(h+1)); every position is visible (the encoder
    memory has no mask).  Per head: softmax(q_h xk_h^T / sqrt(hd)) xv_h, the
    definition `attention` evaluates.  Returns [n_q, d] in fp64.
    """
    q, xk, xv = _f64(q), _f64(xk), _f64(xv)
    d = q.shape[1]
    hd = d // n_head
    out = np.empty_like(q)
    for h in range(n_head):
        c = slice(h * hd, (h + 1) * hd)
        out[:, c] = attention(q[:, c], xk[:, c], xv[:, c])
    return out



def greedy_argmax(logits) -> np.ndarray:
    """Greedy decoding's token choice per row of logits (whisper README,
    "Performance and memory": the argmax over the 51865 logits of a step is
    reduced on the device and only the winning index comes back).

    logits: [rows, n_vocab] (fp32 on the GPU side; widened to fp64, which
    preserves every comparison).  Per row, the definition: the smallest index
    whose value equals the row's maximum.  Readings where the pages say
    nothing: ties go to the smallest index; -0.0 and +0.0 are equal (IEEE
    comparison); a NaN counts as larger than every number, so the first NaN
    wins.  Returns int64 [rows].
    """
    x = _f64(np.atleast_2d(logits))
    out = np.empty(x.shape[0], dtype=np.int64)
    for r in range(x.shape[0]):
        row = x[r]
        nan = np.flatnonzero(np.isnan(row))
        if nan.size:
            out[r] = nan[0]
        else:
            out[r] = np.flatnonzero(row == row.max())[0]
    return out
