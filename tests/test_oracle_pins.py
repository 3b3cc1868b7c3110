"""Pins of the fp64 oracle against facts fixed outside it.

Each test checks the oracle against the pages' shape facts (golden fixtures),
closed forms, invariants, brute-force sums on tiny inputs, or an independent
library implementation (torch float64 layers).  None retypes the oracle's
own formula as its expectation.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests.conftest import read_golden
from tests.torch_reference import torch_encode
from whisper_audio_encoder_amd import synth
from whisper_audio_encoder_amd.configs import CONFIGS, EncoderConfig


# ----------------------------------------------------------------- conv (P-a)
def _brute_conv(x, w, b, stride, pad=1):
    """Pure-Python direct sum over taps and input channels."""
    T_in, C_in = len(x), len(x[0])
    C_out, _, K = w.shape
    T_out = (T_in + 2 * pad - K) // stride + 1
    y = [[0.0] * C_out for _ in range(T_out)]
    for t in range(T_out):
        for o in range(C_out):
            acc = float(b[o])
            for j in range(K):
                src = stride * t + j - pad
                if 0 <= src < T_in:
                    for c in range(C_in):
                        acc += float(w[o, c, j]) * float(x[src][c])
            y[t][o] = acc
    return np.array(y)


@pytest.mark.parametrize("T_in,stride", [(8, 1), (9, 1), (8, 2), (17, 2), (16, 2)])
def test_conv_brute_force(T_in, stride):
    rng = np.random.default_rng(T_in * 10 + stride)
    x = rng.standard_normal((T_in, 3))
    w = rng.standard_normal((4, 3, 3))
    b = rng.standard_normal(4)
    got = oracle.conv1d(x, w, b, stride)
    np.testing.assert_allclose(got, _brute_conv(x, w, b, stride), rtol=0, atol=1e-12)


@pytest.mark.parametrize("stride", [1, 2])
def test_conv_matches_torch(stride):
    rng = np.random.default_rng(7 + stride)
    x = rng.standard_normal((31, 5))
    w = rng.standard_normal((6, 5, 3))
    b = rng.standard_normal(6)
    ref = F.conv1d(torch.from_numpy(x.T[None].copy()), torch.from_numpy(w), torch.from_numpy(b),
                   stride=stride, padding=1)[0].T.numpy()
    np.testing.assert_allclose(oracle.conv1d(x, w, b, stride), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("stride", [1, 2])
def test_conv_delta_input(stride):
    """A unit impulse at (t0, c) reproduces the taps W[:, c, j] at the outputs
    whose window covers t0, and the bias elsewhere (no kernel flip)."""
    T_in, C_in, C_out = 12, 3, 4
    rng = np.random.default_rng(3)
    w = rng.standard_normal((C_out, C_in, 3))
    b = rng.standard_normal(C_out)
    t0, c = 5, 1
    x = np.zeros((T_in, C_in))
    x[t0, c] = 1.0
    y = oracle.conv1d(x, w, b, stride)
    for t in range(y.shape[0]):
        expect = b.copy()
        for j in range(3):
            if stride * t + j - 1 == t0:
                expect = expect + w[:, c, j]
        np.testing.assert_array_equal(y[t], expect)


def test_stem_lengths_golden():
    rows = read_golden("stem_shapes.txt")
    for name, k, s, p, t_in, t_out in rows:
        k, s, p, t_in, t_out = map(int, (k, s, p, t_in, t_out))
        x = np.zeros((t_in, 2))
        w = np.zeros((1, 2, k))
        assert oracle.conv1d(x, w, np.zeros(1), s, pad=p).shape == (t_out, 1), name
    # the general even-length rule of the stride-2 layer
    for t_in in (2, 10, 100, 3000):
        assert oracle.conv1d(np.zeros((t_in, 1)), np.zeros((1, 1, 3)), np.zeros(1), 2).shape[0] == t_in // 2


# ----------------------------------------------------------------- GELU (P-b)
def test_gelu_normal_cdf_golden():
    for xs, phis in read_golden("normal_cdf.txt"):
        x, phi = float(xs), float(phis)
        assert abs(oracle.gelu(x) - x * phi) < 1e-15
        assert abs(oracle.gelu(-x) - (-x) * (1.0 - phi)) < 1e-15


def test_gelu_identities_and_libm():
    x = np.linspace(-9, 9, 2001)
    g = oracle.gelu(x)
    # erf is odd, so gelu(x) - gelu(-x) = x
    np.testing.assert_allclose(g - oracle.gelu(-x), x, rtol=0, atol=1e-14)
    assert oracle.gelu(0.0) == 0.0
    ref = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    np.testing.assert_allclose(g, ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(g, F.gelu(torch.from_numpy(x), approximate="none").numpy(), rtol=0, atol=1e-15)


def test_gelu_is_not_tanh_form():
    x = np.linspace(-6, 6, 4001)
    tanh_form = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.abs(oracle.gelu(x) - tanh_form).max() > 1e-4


# ------------------------------------------------------------ LayerNorm (P-c)
def test_layer_norm_invariants():
    rng = np.random.default_rng(11)
    d, eps = 384, 1e-5
    x = rng.standard_normal((50, d)) * rng.uniform(0.1, 3, (50, 1)) + rng.uniform(-2, 2, (50, 1))
    y = oracle.layer_norm(x, np.ones(d), np.zeros(d), eps)
    assert np.abs(y.mean(axis=1)).max() < 1e-12
    # population variance of the output is sigma^2 / (sigma^2 + eps)
    s2 = x.var(axis=1)
    np.testing.assert_allclose(y.var(axis=1), s2 / (s2 + eps), rtol=1e-12)
    # a constant row normalises to zero, leaving the bias
    beta = rng.standard_normal(d)
    const = oracle.layer_norm(np.full((1, d), 3.25), rng.standard_normal(d), beta, eps)
    np.testing.assert_allclose(const[0], beta, rtol=0, atol=1e-15)


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((33, 96))
    g, b = rng.standard_normal(96), rng.standard_normal(96)
    ref = F.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), torch.from_numpy(b), 1e-5).numpy()
    np.testing.assert_allclose(oracle.layer_norm(x, g, b, 1e-5), ref, rtol=0, atol=1e-13)


# ------------------------------------------------------------ attention (P-d)
def _brute_attention(q, k, v):
    T, hd = q.shape
    out = np.zeros((T, v.shape[1]))
    for t in range(T):
        s = [sum(q[t, e] * k[u, e] for e in range(hd)) / math.sqrt(hd) for u in range(len(k))]
        m = max(s)
        p = [math.exp(x - m) for x in s]
        z = sum(p)
        for u in range(len(k)):
            out[t] += (p[u] / z) * v[u]
    return out


@pytest.mark.parametrize("T", [7, 33])
def test_attention_brute_force(T):
    rng = np.random.default_rng(T)
    q, k, v = (rng.standard_normal((T, 64)) for _ in range(3))
    np.testing.assert_allclose(oracle.attention(q, k, v), _brute_attention(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [7, 33, 130])
def test_attention_matches_torch_sdpa(T):
    rng = np.random.default_rng(100 + T)
    q, k, v = (rng.standard_normal((T, 64)) * 2 for _ in range(3))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a)[None] for a in (q, k, v)))[0].numpy()
    np.testing.assert_allclose(oracle.attention(q, k, v), ref, rtol=0, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    T = 130
    v = rng.standard_normal((T, 64))
    q = rng.standard_normal((T, 64))
    # identical keys, or a zero query: every weight is 1/T
    k_same = np.tile(rng.standard_normal(64), (T, 1))
    np.testing.assert_allclose(oracle.attention(q, k_same, v), np.tile(v.mean(0), (T, 1)), atol=1e-13)
    np.testing.assert_allclose(oracle.attention(np.zeros((T, 64)), rng.standard_normal((T, 64)), v),
                               np.tile(v.mean(0), (T, 1)), atol=1e-13)
    # one key 40 score units above the rest selects its value row
    k = np.zeros((T, 64))
    k[17] = 1.0
    q1 = np.full((1, 64), 40.0 * 8.0 / 64.0)  # q.k / 8 = 40 for key 17, 0 elsewhere
    np.testing.assert_allclose(oracle.attention(q1, k, v)[0], v[17], atol=1e-14)
    # the score matrix rows are probability vectors
    p = oracle.softmax_rows(rng.standard_normal((9, T)) * 10)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)
    assert (p >= 0).all()


def test_attention_permutation_equivariant():
    rng = np.random.default_rng(8)
    T = 40
    q, k, v = (rng.standard_normal((T, 64)) for _ in range(3))
    perm = rng.permutation(T)
    base = oracle.attention(q, k, v)
    np.testing.assert_allclose(oracle.attention(q[perm], k[perm], v[perm]), base[perm], atol=1e-13)
    # permuting keys and values together leaves the output unchanged (no mask, no positions)
    np.testing.assert_allclose(oracle.attention(q, k[perm], v[perm]), base, atol=1e-13)


# ------------------------------------------------------ block / encoder (P-e)
def _small_cfg(**kw):
    base = dict(name="pin", batch=1, n_mels=16, d_model=128, n_head=2, d_ff=512, n_layer=2,
                seed=77, n_frames=40, n_ctx=20)
    base.update(kw)
    return EncoderConfig(**base)


def _small_inputs(cfg, scale_attn=1.0):
    mel, params = synth.make_inputs(cfg)
    params = {k: v.astype(np.float64) for k, v in params.items()}
    for li in range(cfg.n_layer):
        # sharpen the attention so the test is sensitive to the score path
        params[f"l{li}.wq"] *= scale_attn
        params[f"l{li}.wk"] *= scale_attn
    return mel[0].astype(np.float64), params


def test_block_identity_when_outputs_zero():
    cfg = _small_cfg(n_layer=1)
    _, params = _small_inputs(cfg)
    p = {k.split(".", 1)[1]: v for k, v in params.items() if k.startswith("l0.")}
    for f in ("wo", "bo", "fc2_w", "fc2_b"):
        p[f] = np.zeros_like(p[f])
    x = np.random.default_rng(1).standard_normal((cfg.n_ctx, cfg.d_model))
    np.testing.assert_array_equal(oracle.encoder_block(x, p, cfg.n_head, cfg.ln_eps), x)


def test_zero_layers_is_ln_of_stem():
    cfg = _small_cfg(n_layer=0)
    mel, params = _small_inputs(cfg)
    out = oracle.encode(mel, params, 0, cfg.n_head)
    np.testing.assert_allclose(out, torch_encode(mel, params, 0, cfg.n_head), atol=1e-12)


@pytest.mark.parametrize("final_ln", [True, False])
def test_encoder_matches_torch_layers(final_ln):
    cfg = _small_cfg()
    mel, params = _small_inputs(cfg, scale_attn=6.0)
    got = oracle.encode(mel, params, cfg.n_layer, cfg.n_head, cfg.ln_eps, final_ln=final_ln)
    ref = torch_encode(mel, params, cfg.n_layer, cfg.n_head, cfg.ln_eps, final_ln=final_ln)
    assert got.shape == (cfg.n_ctx, cfg.d_model)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)


def test_encoder_taps_consistent():
    cfg = _small_cfg()
    mel, params = _small_inputs(cfg)
    t = oracle.encode(mel, params, cfg.n_layer, cfg.n_head, taps=True)
    assert t["c1"].shape == (cfg.n_frames, cfg.d_model)
    assert t["x0"].shape == (cfg.n_ctx, cfg.d_model)
    assert len(t["blocks"]) == cfg.n_layer
    np.testing.assert_array_equal(t["out"], oracle.encode(mel, params, cfg.n_layer, cfg.n_head))


# ------------------------------------------------- shortened context (drafts)
def test_draft_stem_is_prefix_of_full_stem():
    """A draft of 2T' frames of the same audio gives the full window's stem
    rows 0 .. T'-2 (conv is local and positions are aligned at the start);
    row T'-1 differs, because frame 2T' is the draft's zero padding."""
    cfg = _small_cfg(n_layer=0)
    mel, params = _small_inputs(cfg)
    full = oracle.encode(mel, params, 0, cfg.n_head, taps=True)["x0"]
    for Td in (1, 2, 7, 13):
        draft = oracle.encode(mel[:2 * Td], params, 0, cfg.n_head, taps=True)["x0"]
        assert draft.shape == (Td, cfg.d_model)
        np.testing.assert_allclose(draft[:Td - 1], full[:Td - 1], rtol=0, atol=1e-12)
        assert np.abs(draft[Td - 1] - full[Td - 1]).max() > 1e-4


def test_draft_positions_are_leading_rows():
    """With the stem silenced (zero conv weights and biases, gelu(0) = 0) and
    no blocks, a draft's output is exactly rows 0 .. T'-1 of the table."""
    cfg = _small_cfg(n_layer=0)
    mel, params = _small_inputs(cfg)
    for f in ("conv1_w", "conv1_b", "conv2_w", "conv2_b"):
        params[f] = np.zeros_like(params[f])
    out = oracle.encode(mel[:14], params, 0, cfg.n_head, final_ln=False)
    np.testing.assert_array_equal(out, params["pos"][:7])


def test_draft_matches_torch_layers():
    """Blocks over T' < n_ctx positions against torch's float64 layers."""
    cfg = _small_cfg()
    mel, params = _small_inputs(cfg, scale_attn=6.0)
    got = oracle.encode(mel[:22], params, cfg.n_layer, cfg.n_head, cfg.ln_eps)
    ref = torch_encode(mel[:22], params, cfg.n_layer, cfg.n_head, cfg.ln_eps)
    assert got.shape == (11, cfg.d_model)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)


def test_draft_longer_than_table_is_refused():
    cfg = _small_cfg(n_layer=0)
    mel, params = _small_inputs(cfg)
    longer = np.concatenate([mel, mel[:4]])
    with pytest.raises(AssertionError):
        oracle.encode(longer, params, 0, cfg.n_head)


# ------------------------------------------- cross-attention K/V (decoder side)
def test_cross_kv_brute_force():
    """Pure-Python sums at a tiny, non-square-friendly size."""
    rng = np.random.default_rng(21)
    T, d = 5, 6
    m = rng.standard_normal((T, d))
    wk, wv, bv = rng.standard_normal((d, d)), rng.standard_normal((d, d)), rng.standard_normal(d)
    K, V = oracle.cross_kv(m, wk, wv, bv)
    for t in range(T):
        for o in range(d):
            k_ref = sum(float(m[t, c]) * float(wk[o, c]) for c in range(d))
            v_ref = float(bv[o]) + sum(float(m[t, c]) * float(wv[o, c]) for c in range(d))
            assert abs(K[t, o] - k_ref) < 1e-12 and abs(V[t, o] - v_ref) < 1e-12


def test_cross_kv_matches_torch_linear_and_identity():
    rng = np.random.default_rng(22)
    m = rng.standard_normal((37, 64))
    wk, wv, bv = rng.standard_normal((64, 64)), rng.standard_normal((64, 64)), rng.standard_normal(64)
    K, V = oracle.cross_kv(m, wk, wv, bv)
    tm = torch.from_numpy(m)
    np.testing.assert_allclose(K, F.linear(tm, torch.from_numpy(wk)).numpy(), atol=1e-12)
    np.testing.assert_allclose(V, F.linear(tm, torch.from_numpy(wv), torch.from_numpy(bv)).numpy(), atol=1e-12)
    eye = np.eye(64)
    K, V = oracle.cross_kv(m, eye, eye, bv)
    np.testing.assert_array_equal(K, m)
    np.testing.assert_allclose(V, m + bv, atol=0)


def test_cross_k_bias_would_be_unobservable():
    """x_wk has no bias; a bias c would add q.c to every score of a query,
    which the softmax over keys cancels: the zero-bias reading loses nothing."""
    rng = np.random.default_rng(23)
    m = rng.standard_normal((30, 64))
    wk = rng.standard_normal((64, 64)) * 0.1
    K, _ = oracle.cross_kv(m, wk, wk, np.zeros(64))
    q = rng.standard_normal((3, 64))
    c = rng.standard_normal(64)
    np.testing.assert_allclose(oracle.softmax_rows(q @ (K + c).T), oracle.softmax_rows(q @ K.T), atol=1e-12)


# ---------------------------------------- decode-step cross-attention (one query)
def test_cross_attend_brute_force():
    """Pure-Python softmax over keys per head at a tiny size (2 heads of 4
    dims, 5 keys, 2 query rows), with the 1/sqrt(hd) scale written out."""
    rng = np.random.default_rng(31)
    n_q, T, H, hd = 2, 5, 2, 4
    q = rng.standard_normal((n_q, H * hd))
    k = rng.standard_normal((T, H * hd))
    v = rng.standard_normal((T, H * hd))
    out = oracle.cross_attend(q, k, v, H)
    for i in range(n_q):
        for h in range(H):
            cols = range(h * hd, (h + 1) * hd)
            s = [sum(float(q[i, c]) * float(k[u, c]) for c in cols) / math.sqrt(hd) for u in range(T)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for c in cols:
                ref = sum(e[u] / z * float(v[u, c]) for u in range(T))
                assert abs(out[i, c] - ref) < 1e-12


def test_cross_attend_matches_torch_sdpa():
    """torch's scaled_dot_product_attention (fp64, no mask) per head, at the
    decode-step shape: one query row over 1500 keys, 20 heads of 64."""
    rng = np.random.default_rng(32)
    T, H = 1500, 20
    q = rng.standard_normal((1, 64 * H))
    k = rng.standard_normal((T, 64 * H))
    v = rng.standard_normal((T, 64 * H))
    out = oracle.cross_attend(q, k, v, H)
    tq = torch.from_numpy(q).view(1, H, 64).transpose(0, 1)
    tk = torch.from_numpy(k).view(T, H, 64).transpose(0, 1)
    tv = torch.from_numpy(v).view(T, H, 64).transpose(0, 1)
    ref = F.scaled_dot_product_attention(tq, tk, tv).transpose(0, 1).reshape(1, 64 * H)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_cross_attend_closed_forms():
    """One key: the output is that key's value row.  Identical keys: the mean
    of the values.  A +40 score margin on one key selects its value row.
    Heads and query rows are independent of each other."""
    rng = np.random.default_rng(33)
    H, d = 3, 192
    q = rng.standard_normal((2, d))
    v = rng.standard_normal((7, d))
    np.testing.assert_allclose(oracle.cross_attend(q, rng.standard_normal((1, d)), v[:1], H), np.repeat(v[:1], 2, 0), atol=1e-15)
    same = np.repeat(rng.standard_normal((1, d)), 7, 0)
    np.testing.assert_allclose(oracle.cross_attend(q, same, v, H), np.repeat(v.mean(0, keepdims=True), 2, 0), atol=1e-13)
    k = np.zeros((7, d))
    qq = np.zeros((1, d))
    qq[0, :64] = 1.0
    k[4, :64] = 40 * 8 / 64  # head 0: key 4 scores 40, the others 0
    got = oracle.cross_attend(qq, k, v, H)
    np.testing.assert_allclose(got[0, :64], v[4, :64], atol=1e-15)
    k2 = rng.standard_normal((7, d))
    k3 = k2.copy()
    k3[:, 64:128] = rng.standard_normal((7, 64))  # change head 1's keys only
    a, b = oracle.cross_attend(q, k2, v, H), oracle.cross_attend(q, k3, v, H)
    np.testing.assert_array_equal(a[:, :64], b[:, :64])
    np.testing.assert_array_equal(a[:, 128:], b[:, 128:])
    assert not np.allclose(a[:, 64:128], b[:, 64:128])
    np.testing.assert_allclose(oracle.cross_attend(q[1:], k2, v, H), a[1:], rtol=1e-13, atol=1e-14)


def test_greedy_argmax_brute_force():
    """A pure-Python scan (keep the first strictly larger value) over small
    integer-valued rows, where ties are common."""
    rng = np.random.default_rng(41)
    x = rng.integers(-2, 3, size=(50, 9)).astype(np.float32)
    got = oracle.greedy_argmax(x)
    for r in range(x.shape[0]):
        best = 0
        for i in range(1, x.shape[1]):
            if float(x[r, i]) > float(x[r, best]):
                best = i
        assert got[r] == best


def test_greedy_argmax_matches_numpy():
    """numpy.argmax (first occurrence of the maximum; a NaN wins at its
    first position) at the decode shape: 16 rows of 51865 fp32 logits, with
    planted ties and NaNs."""
    rng = np.random.default_rng(42)
    x = (4 * rng.standard_normal((16, 51865))).astype(np.float32)
    x[3, [100, 7000, 51864]] = 99.0
    x[5, 40000] = np.nan
    x[6, [10, 20]] = np.nan
    x[7] = x[7].max()
    np.testing.assert_array_equal(oracle.greedy_argmax(x), np.argmax(x, axis=1))
    assert oracle.greedy_argmax(x)[3] == 100


def test_greedy_argmax_closed_forms():
    """Constant, one-hot, monotone rows; signed zeros compare equal; -inf and
    +inf; NaN beats everything; adjacent fp32 values are told apart; the
    largest finite and the smallest subnormal magnitudes."""
    f = np.float32
    cases = [
        (np.full(7, 1.5, f), 0),
        (np.eye(1, 11, 6, dtype=f)[0], 6),
        (np.arange(13, dtype=f), 12),
        (np.arange(13, dtype=f)[::-1].copy(), 0),
        (np.array([-0.0, 0.0], f), 0),
        (np.array([0.0, -0.0], f), 0),
        (np.array([-1.0, -0.0, 0.0], f), 1),
        (np.full(5, -np.inf, f), 0),
        (np.array([-np.inf, np.inf, np.inf], f), 1),
        (np.array([1e30, 2.0, 3e38, np.nan, 5.0], f), 3),
        (np.array([np.nan, np.nan], f), 0),
        (np.array([1.0, np.nextafter(f(1.0), f(2.0))], f), 1),
        (np.array([-3e38, 3.4e38, -np.inf], f), 1),
        (np.array([0.0, 1e-45, -1e-45], f), 1),
    ]
    for row, want in cases:
        assert oracle.greedy_argmax(row[None])[0] == want, (row, want)
    assert oracle.greedy_argmax(np.zeros((0, 4), f)).shape == (0,)


# --------------------------------------------------------------- shapes (P-f)
def test_family_golden_matches_configs():
    fam = {r[0]: tuple(map(int, r[1:])) for r in read_golden("whisper_family.txt")}
    pairs = {"c1": "tiny", "c2": "base", "c3": "small", "c4": "large-v3"}
    for cname, fname in pairs.items():
        c = CONFIGS[cname]
        assert (c.n_layer, c.d_model, c.n_head, c.n_mels) == fam[fname], cname
        assert c.d_model // c.n_head == 64 and c.d_ff == 4 * c.d_model
    c0 = CONFIGS["c0"]
    assert (c0.d_model, c0.n_head, c0.n_mels, c0.n_layer) == (384, 6, 80, 1)


def test_full_window_shape():
    """3000 x n_mels in, 1500 x d out, for a full-length window (one block)."""
    cfg = CONFIGS["c0"]
    mel, params = synth.make_inputs(cfg)
    out = oracle.encode(mel[0], params, cfg.n_layer, cfg.n_head, cfg.ln_eps)
    assert mel.shape == (1, 3000, 80) and out.shape == (1500, 384)
    assert np.isfinite(out).all()
