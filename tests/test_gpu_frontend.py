"""The log-mel frontend on the GPU (wenc_log_mel through the C ABI) against
the fp64 oracle (oracle/frontend.py), and audio -> log-mel -> encoder end to
end.

Inputs are synthetic 16 kHz windows from synth.make_audio: an 11-s
speech-like stretch (harmonic series on a 90-250 Hz fundamental under random
envelopes, silent gaps, light noise) padded with zeros to the 30-s window,
standing in for the pages' clips (CKE page, "The Frontend").

Tolerance, from the arithmetic: the GPU's STFT is a 20 x 20 FFT in fp32 (two
stages of 20-term sums and a twiddle product per bin), so a bin's error is
about 1e-7 of the frame's peak amplitude; the clamp keeps only bins within
80 dB (a factor 1e-4 in amplitude) of the peak, whose relative power error is
then at most a few 1e-3 in the worst bin, i.e. about 1e-3 in log10 before
the mel sum averages it and 3e-4 after the / 4 at worst; in practice the
filters sum several bins and the error is far smaller.  The bar is 1e-4
absolute on every value.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, check_encoder_tolerance, dev, host, say
from tests.test_gpu_encoder import encoder, inputs
from whisper_audio_encoder_amd import synth, wenc
from whisper_audio_encoder_amd.configs import CONFIGS

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _check(got, audio, n_mels, what):
    ref = oracle.log_mel(audio, n_mels)
    err = np.abs(got.astype(np.float64) - ref).max()
    say(f"{what}: max abs err {err:.2e}")
    assert got.shape == ref.shape and err <= TOL, what


@pytest.mark.parametrize("name,batch", [("c1", 3), ("c4", 4)])   # 80 and 128 mel bins
def test_log_mel_matches_oracle(name, batch):
    cfg = CONFIGS[name]
    say(f"log-mel {name} n_mels {cfg.n_mels} batch {batch}")
    audio = synth.make_audio(batch, seed=cfg.seed)
    mel = host(encoder(name).log_mel(dev(audio)))
    assert mel.shape == (batch, 3000, cfg.n_mels)
    for b in range(batch):
        _check(mel[b], audio[b], cfg.n_mels, f"{name} window {b}")


def test_log_mel_loud_tone_and_silence():
    """A full-scale tone (the clamp bites in most bins) and silence (all -1.5)."""
    n = 480000
    tone = np.cos(2 * np.pi * 1234.5 * np.arange(n) / 16000).astype(np.float32)
    silent = np.zeros(n, dtype=np.float32)
    say("log-mel tone and silence")
    mel = host(encoder("c0").log_mel(dev(np.stack([tone, silent]))))
    _check(mel[0], tone, 80, "tone")
    assert np.abs(mel[1] + 1.5).max() <= 1e-6


@pytest.mark.parametrize("F", [2, 34, 64])
def test_log_mel_short_windows(F):
    """Windows of F frames: reflection at both ends of a short signal, and a
    partial last 32-frame tile (34 = 32 + 2)."""
    cfg = CONFIGS["c0"].with_(n_frames=F, n_ctx=F // 2, name=f"F{F}")
    e = wenc.Encoder(cfg, synth.pack_blob(cfg, synth.make_params(np.random.default_rng(0), cfg)))
    try:
        a = synth.make_audio(2, n_samples=160 * F, seed=F, speech_s=0.25)
        say(f"log-mel {F} frames")
        mel = host(e.log_mel(dev(a)))
        for b in range(2):
            _check(mel[b], a[b], 80, f"{F} frames, window {b}")
    finally:
        e.close()


@pytest.mark.parametrize("n_mels", [8, 24, 64])
def test_log_mel_narrow_filter_banks(n_mels):
    """Few filters: each triangle spans more than 16 bins (up to 99 at 8
    filters), so the kernel reads it through several 16-bin windows."""
    cfg = CONFIGS["c0"].with_(n_mels=n_mels, name=f"m{n_mels}")
    e = wenc.Encoder(cfg, synth.pack_blob(cfg, synth.make_params(np.random.default_rng(0), cfg)))
    try:
        a = synth.make_audio(2, seed=n_mels)
        say(f"log-mel {n_mels} filters")
        mel = host(e.log_mel(dev(a)))
        for b in range(2):
            _check(mel[b], a[b], n_mels, f"{n_mels} filters, window {b}")
    finally:
        e.close()


def test_log_mel_chunking_is_bitwise():
    name = "c2"
    cfg, _, _, blob = inputs(name)
    audio = dev(synth.make_audio(5, seed=11))
    say("log-mel chunking c2 max_batch 2")
    small = wenc.Encoder(cfg, blob, max_batch=2)
    try:
        a = host(small.log_mel(audio))
    finally:
        small.close()
    assert np.array_equal(a, host(encoder(name).log_mel(audio)))


def test_audio_to_encoder_output():
    """audio -> wenc_log_mel -> wenc_forward against oracle.log_mel -> oracle.encode."""
    name = "c1"
    cfg, _, params, _ = inputs(name)
    audio = synth.make_audio(1, seed=42)
    say("audio -> log-mel -> encoder, c1")
    enc = encoder(name)
    out = host(enc.forward(enc.log_mel(dev(audio))))[0]
    ref = oracle.encode(oracle.log_mel(audio[0], cfg.n_mels).astype(np.float32), params, cfg.n_layer, cfg.n_head,
                        cfg.ln_eps, bool(cfg.final_ln))
    check_encoder_tolerance(out, ref, "audio to encoder c1")


def test_log_mel_errors():
    cfg, _, _, blob = inputs("c0")
    say("log-mel error paths")
    h = encoder("c0").h
    audio = torch.zeros((1, 480000), device=DEV)
    mel = torch.empty((1, 3000, 80), device=DEV)
    with pytest.raises(wenc.WencError) as e:
        wenc.wenc_log_mel(h, audio, -1, mel)
    assert e.value.code == wenc.WENC_EINVAL
    wenc.wenc_log_mel(h, audio, 0, mel)  # empty batch: a no-op
    wide = cfg.with_(n_mels=136, name="m136")
    e2 = wenc.Encoder(wide, synth.pack_blob(wide, synth.make_params(np.random.default_rng(0), wide)))
    try:
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_log_mel(e2.h, audio, 1, torch.empty((1, 3000, 136), device=DEV))
        assert e.value.code == wenc.WENC_EINVAL and "n_mels" in str(e.value)
    finally:
        e2.close()
