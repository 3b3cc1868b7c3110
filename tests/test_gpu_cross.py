"""Cross-attention K/V of the decoder layers on the GPU (wenc_load_cross +
wenc_prepare_cross through the C ABI), and the KV-split GEMM epilogue.

The decoder projects the frozen encoder memory into per-layer keys and
values once per clip (whisper 0.9.0 API page, wh_prepare_cross; model.nu:
x_wk has no bias).  End to end, the memory is the library's own encoder
output; the oracle side projects the fp64 oracle memory.  A second check
isolates the projection: the GPU K/V against an fp64 product of the fp16
memory the kernel consumed.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, check_encoder_tolerance, dev, f16_dev, host, row_cosine, say
from tests.test_gpu_encoder import encoder, inputs, oracle_out
from tests.test_gpu_kernels import _gemm
from whisper_audio_encoder_amd import synth, wenc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,d", [(1, 64), (300, 384), (1537, 512), (24000, 1280)])
def test_gemm_kv_split(M, d):
    say(f"gemm KV M={M} d={d}")
    rng = np.random.default_rng(M + d)
    A = rng.standard_normal((M, d)).astype(np.float16)
    W = (0.05 * rng.standard_normal((2 * d, d))).astype(np.float16)
    b = np.concatenate([np.zeros(d), 0.1 * rng.standard_normal(d)]).astype(np.float32)
    C = torch.full((M, d), float("nan"), dtype=torch.float16, device=DEV)
    C2 = torch.full((M, d), float("nan"), dtype=torch.float16, device=DEV)
    _gemm(f16_dev(A), f16_dev(W), dev(b), wenc.WENC_EPI_KV, M, 2 * d, d, C=C, C2=C2, ldc=d, n_split=d)
    ref = A.astype(np.float64) @ W.astype(np.float64).T + b
    np.testing.assert_allclose(host(C).astype(np.float64), ref[:, :d], rtol=1e-3, atol=1e-4)
    np.testing.assert_allclose(host(C2).astype(np.float64), ref[:, d:], rtol=1e-3, atol=1e-4)


N_DEC = {"c1": 4, "c2": 6, "c3": 12, "c4": 32}   # the Whisper family's decoders are as deep as their encoders
ITEMS = {"c1": [0], "c2": [0, 7], "c3": [0, 15], "c4": [0, 15]}


def _loaded(name, enc=None):
    cfg, _, _, _ = inputs(name)
    n = N_DEC[name]
    cross = synth.make_cross_params(cfg, n)
    enc = enc or encoder(name)
    enc.load_cross(synth.pack_cross_blob(cfg, cross, n), n)
    return cfg, cross, enc


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_cross_kv_matches_oracle(name):
    cfg, cross, enc = _loaded(name)
    _, mel, _, _ = inputs(name)
    n = N_DEC[name]
    say(f"cross K/V {name}: {n} decoder layers, batch {cfg.batch}")
    memory = enc.forward(dev(mel))
    xk, xv = enc.prepare_cross(memory)
    mem_h, xk_h, xv_h = host(memory), host(xk), host(xv)
    assert xk_h.shape == (n, cfg.batch, cfg.n_ctx, cfg.d_model) and np.isfinite(xk_h).all() and np.isfinite(xv_h).all()
    layers = sorted({0, n // 2, n - 1})
    for it in ITEMS[name]:
        ref_mem = oracle_out(name, it)
        m16 = mem_h[it].astype(np.float16).astype(np.float64)  # what the kernel consumed
        for l in layers:
            p = [cross[f"d{l}.{f}"] for f in synth.CROSS_FIELDS]
            K, V = oracle.cross_kv(ref_mem, *p)
            check_encoder_tolerance(xk_h[l, it], K, f"{name} item {it} layer {l} K")
            check_encoder_tolerance(xv_h[l, it], V, f"{name} item {it} layer {l} V")
            K16, V16 = oracle.cross_kv(m16, *p)
            np.testing.assert_allclose(xk_h[l, it].astype(np.float64), K16, rtol=2e-3, atol=2e-4)
            np.testing.assert_allclose(xv_h[l, it].astype(np.float64), V16, rtol=2e-3, atol=2e-4)


def test_cross_kv_of_a_draft():
    name = "c2"
    cfg, cross, enc = _loaded(name)
    _, mel, _, _ = inputs(name)
    Td = 500
    say(f"cross K/V of drafts, {name} n_ctx {Td}")
    memory = enc.forward(dev(np.ascontiguousarray(mel[:, :2 * Td])), n_ctx=Td)
    xk, xv = enc.prepare_cross(memory)
    assert xk.shape == (N_DEC[name], cfg.batch, Td, cfg.d_model)
    mem_h, xk_h, xv_h = host(memory), host(xk), host(xv)
    for l in (0, N_DEC[name] - 1):
        p = [cross[f"d{l}.{f}"] for f in synth.CROSS_FIELDS]
        K, V = oracle.cross_kv(mem_h[3].astype(np.float16).astype(np.float64), *p)
        assert row_cosine(xk_h[l, 3], K).min() >= 0.9999 and row_cosine(xv_h[l, 3], V).min() >= 0.9999


def test_cross_kv_chunking_is_bitwise():
    name = "c2"
    cfg, _, _, blob = inputs(name)
    say("cross K/V chunking c2 max_batch 3")
    _, _, big = _loaded(name)
    small = wenc.Encoder(cfg, blob, max_batch=3)
    try:
        _loaded(name, small)
        memory = big.forward(dev(inputs(name)[1]))
        a = [host(t) for t in big.prepare_cross(memory)]
        b = [host(t) for t in small.prepare_cross(memory)]
    finally:
        small.close()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_cross_errors():
    cfg, _, _, blob = inputs("c0")
    say("cross K/V error paths")
    enc = wenc.Encoder(cfg, blob)
    try:
        mem = torch.zeros((1, cfg.n_ctx, cfg.d_model), device=DEV)
        xk = torch.empty((1, 1, cfg.n_ctx, cfg.d_model), dtype=torch.float16, device=DEV)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_prepare_cross(enc.h, mem, 1, cfg.n_ctx, xk, xk)
        assert e.value.code == wenc.WENC_ESTATE
        cross = synth.make_cross_params(cfg, 1)
        blob_x = synth.pack_cross_blob(cfg, cross, 1)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_load_cross(enc.h, 1, blob_x[:-2])
        assert e.value.code == wenc.WENC_EINVAL and "exactly" in str(e.value)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_load_cross(enc.h, 0, blob_x)
        assert e.value.code == wenc.WENC_EINVAL
        enc.load_cross(blob_x, 1)
        xv = torch.empty_like(xk)
        for bad in (0, cfg.n_ctx + 1):
            with pytest.raises(wenc.WencError) as e:
                wenc.wenc_prepare_cross(enc.h, mem, 1, bad, xk, xv)
            assert e.value.code == wenc.WENC_EINVAL
        wenc.wenc_prepare_cross(enc.h, mem, 0, cfg.n_ctx, xk, xv)  # empty batch: a no-op
        # zero memory: K = 0 and V = x_bv exactly
        wenc.wenc_prepare_cross(enc.h, mem, 1, cfg.n_ctx, xk, xv)
        assert not host(xk).any()
        assert np.array_equal(host(xv)[0, 0], np.broadcast_to(cross["d0.x_bv"], (cfg.n_ctx, cfg.d_model)))
        # reloading replaces the previous weights (a different depth and values)
        cross2 = synth.make_cross_params(cfg, 2)
        cross2 = {k: (v + np.float16(0.5)).astype(np.float16) for k, v in cross2.items()}
        enc.load_cross(synth.pack_cross_blob(cfg, cross2, 2), 2)
        xk2 = torch.empty((2, 1, cfg.n_ctx, cfg.d_model), dtype=torch.float16, device=DEV)
        xv2 = torch.empty_like(xk2)
        wenc.wenc_prepare_cross(enc.h, mem, 1, cfg.n_ctx, xk2, xv2)
        for layer in range(2):
            assert not host(xk2[layer]).any()
            assert np.array_equal(host(xv2)[layer, 0],
                                  np.broadcast_to(cross2[f"d{layer}.x_bv"], (cfg.n_ctx, cfg.d_model)))
    finally:
        enc.close()
