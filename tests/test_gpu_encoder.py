"""End-to-end parity on the GPU: wenc_forward through the C ABI against the
fp64 oracle on the five seeded workloads, plus stage taps, determinism,
batch invariance, chunking, poisoned scratch and the error paths.

Every workload runs at its full batch in the same launch configuration the
benchmark times; the oracle checks every item of the small workloads and a
sample of items (the first and the last) of the two largest, whose fp64
windows cost seconds each on the host.
"""
import functools
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, check_encoder_tolerance, dev, host, row_cosine, say
from whisper_audio_encoder_amd import synth, wenc
from whisper_audio_encoder_amd.configs import CONFIGS

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def inputs(name):
    cfg = CONFIGS[name]
    mel, params = synth.make_inputs(cfg)
    return cfg, mel, params, synth.pack_blob(cfg, params)


@functools.lru_cache(maxsize=None)
def oracle_out(name, item, taps=False):
    cfg, mel, params, _ = inputs(name)
    return oracle.encode(mel[item], params, cfg.n_layer, cfg.n_head, cfg.ln_eps, bool(cfg.final_ln), taps=taps)


@functools.lru_cache(maxsize=None)
def encoder(name, max_batch=None):
    cfg, _, _, blob = inputs(name)
    return wenc.Encoder(cfg, blob, max_batch=max_batch)


ITEMS = {"c0": [0], "c1": [0], "c2": list(range(8)), "c3": [0, 15], "c4": [0, 15]}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_encoder_matches_oracle(name):
    cfg, mel, _, _ = inputs(name)
    say(f"encoder {name} batch {cfg.batch}")
    out = host(encoder(name).forward(dev(mel)))
    assert out.shape == (cfg.batch, cfg.n_ctx, cfg.d_model)
    assert np.isfinite(out).all()
    for it in ITEMS[name]:
        check_encoder_tolerance(out[it], oracle_out(name, it), f"{name} item {it}")


def test_stage_taps_c0():
    """conv1, stem and block outputs of the c0 workload against the oracle's
    stage values (relative error per tensor <= 1e-2)."""
    name = "c0"
    cfg, mel, _, _ = inputs(name)
    say("taps c0")
    enc = encoder(name)
    m = dev(mel)
    ref = oracle_out(name, 0, taps=True)
    c1 = host(enc.tap(m, wenc.WENC_TAP_C1))[0].astype(np.float64)
    stem = host(enc.tap(m, wenc.WENC_TAP_STEM))[0]
    blk = host(enc.tap(m, wenc.WENC_TAP_BLOCK + 0))[0]
    for got, want, what in [(c1, ref["c1"], "c1"), (stem, ref["x0"], "stem"), (blk, ref["blocks"][0], "block0")]:
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        say(f"tap {what}: relative error {rel:.2e}")
        assert rel <= 1e-2, what
        assert row_cosine(got, want).min() >= 0.9999, what


def test_deterministic_and_batch_invariant():
    name = "c2"
    cfg, mel, _, _ = inputs(name)
    say("determinism / batch invariance c2")
    enc = encoder(name)
    m = dev(mel)
    a = host(enc.forward(m))
    b = host(enc.forward(m))
    assert np.array_equal(a, b)
    single = host(enc.forward(dev(mel[3:4])))
    assert np.array_equal(single[0], a[3])


def test_chunking_matches_full_batch():
    name = "c2"
    cfg, mel, _, blob = inputs(name)
    say("chunking c2 max_batch 3")
    full = host(encoder(name).forward(dev(mel)))
    small = wenc.Encoder(cfg, blob, max_batch=3)
    try:
        chunked = host(small.forward(dev(mel)))
    finally:
        small.close()
    assert np.array_equal(full, chunked)


def test_poisoned_scratch_gives_same_output(monkeypatch):
    """Scratch filled with NaN at creation: no kernel may read what it did not write."""
    name = "c1"
    cfg, mel, _, blob = inputs(name)
    say("poisoned scratch c1")
    monkeypatch.setenv("WENC_POISON_SCRATCH", "1")
    enc = wenc.Encoder(cfg, blob)
    try:
        out = host(enc.forward(dev(mel)))
    finally:
        enc.close()
    assert np.array_equal(out, host(encoder(name).forward(dev(mel))))


def test_non_finite_input_propagates_within_its_window():
    """A NaN or an infinity in one window's mel is not sanitised: that
    window's whole memory becomes NaN (every position attends to the
    poisoned keys), as in the oracle, and the other windows' outputs keep
    every bit."""
    name = "c2"
    cfg, mel, params, _ = inputs(name)
    say("non-finite mel c2")
    enc = encoder(name)
    clean = host(enc.forward(dev(mel)))
    bad = mel.copy()
    bad[2, 1234, 17] = np.nan
    bad[5, 2999, 0] = np.inf
    out = host(enc.forward(dev(bad)))
    for b in (2, 5):
        assert np.isnan(out[b]).all(), b
    for b in (0, 1, 3, 4, 6, 7):
        assert np.array_equal(out[b], clean[b]), b
    small = CONFIGS["c0"]
    m0, p0 = synth.make_inputs(small)
    m0 = m0.copy()
    m0[0, 1234, 17] = np.nan
    ref = oracle.encode(m0[0], p0, small.n_layer, small.n_head)
    assert np.isnan(ref).all()


def test_debug_sync_mode_gives_same_output(monkeypatch):
    """WENC_DEBUG_SYNC=1 (a stream synchronise and error check after every
    launch) changes no result bit and reports success."""
    name = "c1"
    cfg, mel, _, blob = inputs(name)
    say("debug sync c1")
    monkeypatch.setenv("WENC_DEBUG_SYNC", "1")
    enc = wenc.Encoder(cfg, blob)
    try:
        out = host(enc.forward(dev(mel)))
    finally:
        enc.close()
    assert np.array_equal(out, host(encoder(name).forward(dev(mel))))


def test_no_final_ln_and_zero_layers():
    base = CONFIGS["c0"]
    rng_cfg = base.with_(n_layer=0, final_ln=0, name="c0-l0")
    mel, params = synth.make_inputs(rng_cfg)
    say("zero layers, no final LN")
    enc = wenc.Encoder(rng_cfg, synth.pack_blob(rng_cfg, params))
    try:
        out = host(enc.forward(dev(mel)))[0]
    finally:
        enc.close()
    ref = oracle.encode(mel[0], params, 0, rng_cfg.n_head, final_ln=False)
    check_encoder_tolerance(out, ref, "L=0 no final LN")


def test_error_paths():
    cfg, mel, _, blob = inputs("c0")
    say("error paths")
    h = wenc.wenc_create(wenc.make_config(cfg))
    try:
        m = dev(mel)
        out = torch.empty((1, cfg.n_ctx, cfg.d_model), device=DEV)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_forward(h, m, 1, out)
        assert e.value.code == wenc.WENC_ESTATE
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_load(h, blob[:-2])
        assert e.value.code == wenc.WENC_EINVAL and "exactly" in str(e.value)
        wenc.wenc_load(h, blob)
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_forward(h, m, -1, out)
        assert e.value.code == wenc.WENC_EINVAL
        wenc.wenc_forward(h, m, 0, out)  # empty batch: a no-op
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_forward_tap(h, m, 1, wenc.WENC_TAP_BLOCK + cfg.n_layer, out)
        assert e.value.code == wenc.WENC_EINVAL
    finally:
        wenc.wenc_destroy(h)


def test_enomem_reports_free_memory():
    # fc1 activations of 2000 windows at d_ff 65536: ~390 GB, beyond any one GPU
    cfg = CONFIGS["c4"].with_(n_layer=1, d_ff=65536)
    say("enomem")
    big = wenc.make_config(cfg, max_batch=2000)
    import ctypes
    h = ctypes.c_void_p()
    rc = wenc.lib().wenc_create(ctypes.byref(big), ctypes.byref(h))
    assert rc == wenc.WENC_ENOMEM and h.value is None
    msg = wenc.wenc_last_error()
    assert "cannot allocate" in msg and "free" in msg
