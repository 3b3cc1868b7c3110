"""Pins of the fp64 log-mel oracle (oracle/frontend.py) against facts fixed
outside it: torch's STFT, Hugging Face's Whisper feature extractor and mel
filter bank (the implementation the CKE page checks its frontend against),
the Slaney scale's defining points, a pure tone's closed-form spectrum, and
invariants of the clamp and rescale.
"""
import numpy as np
import pytest
import torch

import oracle
from whisper_audio_encoder_amd import synth


def _audio(n=480000, seed=1):
    return synth.make_audio(1, n_samples=n, seed=seed)[0]


def test_stft_matches_torch_stft():
    x = _audio(16000 * 3)
    got = oracle.stft_power(x)
    X = torch.stft(torch.from_numpy(x.astype(np.float64)), n_fft=400, hop_length=160,
                   window=torch.hann_window(400, periodic=True, dtype=torch.float64),
                   center=True, pad_mode="reflect", return_complex=True)
    ref = (X.abs() ** 2).numpy().T[:-1]  # torch keeps the last frame; the window has 3000 of 3001
    assert got.shape == (300, 201) == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12 * ref.max())


def test_pure_tone_closed_form():
    """A cosine of amplitude A on bin k0 = 50 (2 kHz): the periodic Hann's
    spectrum is -N/4, N/2, -N/4 on bins k0-1, k0, k0+1 (times A/2), zero
    elsewhere, so interior frames carry power (A N / 4)^2 on k0 and
    (A N / 8)^2 on its neighbours."""
    A, k0, n = 0.3, 50, 16000
    x = A * np.cos(2 * np.pi * k0 * np.arange(n) / 400.0)
    p = oracle.stft_power(x)[5:-5]
    np.testing.assert_allclose(p[:, k0], (A * 400 / 4) ** 2, rtol=1e-9)
    np.testing.assert_allclose(p[:, k0 - 1], (A * 400 / 8) ** 2, rtol=1e-9)
    np.testing.assert_allclose(p[:, k0 + 1], (A * 400 / 8) ** 2, rtol=1e-9)
    others = np.delete(p, [k0 - 1, k0, k0 + 1], axis=1)
    assert others.max() < 1e-18 * p[:, k0].max() + 1e-20


def test_slaney_scale_points():
    m = oracle.frontend.hz_to_mel_slaney([0.0, 1000.0, 6400.0, 500.0])
    np.testing.assert_allclose(m, [0.0, 15.0, 42.0, 7.5], rtol=1e-12, atol=1e-12)
    f = np.linspace(0, 8000, 57)
    np.testing.assert_allclose(oracle.frontend.mel_to_hz_slaney(oracle.frontend.hz_to_mel_slaney(f)), f,
                               rtol=1e-12, atol=1e-9)


@pytest.mark.parametrize("n_mels", [80, 128])
def test_mel_filters_match_hf_and_have_unit_area(n_mels):
    from transformers.audio_utils import mel_filter_bank
    got = oracle.mel_filters(n_mels)
    ref = mel_filter_bank(num_frequency_bins=201, num_mel_filters=n_mels, min_frequency=0.0,
                          max_frequency=8000.0, sampling_rate=16000, norm="slaney", mel_scale="slaney").T
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12)
    # the continuous triangles have unit area; the 40-Hz bin sum approximates it for wide filters
    wide = np.count_nonzero(got, axis=1) >= 6
    assert wide.sum() >= 20
    np.testing.assert_allclose(got[wide].sum(axis=1) * 40.0, 1.0, rtol=0.025)


@pytest.mark.parametrize("n_mels", [80, 128])
def test_log_mel_matches_hf_feature_extractor(n_mels):
    from transformers import WhisperFeatureExtractor
    x = _audio(seed=3 + n_mels)
    got = oracle.log_mel(x, n_mels)
    fe = WhisperFeatureExtractor(feature_size=n_mels)
    ref = fe(x, sampling_rate=16000, return_tensors="np")["input_features"][0].T
    assert got.shape == ref.shape == (3000, n_mels)
    # HF computes in float32; the pages report max |d| = 1.8e-5 for their own check
    assert np.abs(got - ref).max() < 1e-4


def test_silence_and_scaling_invariants():
    z = np.zeros(48000)
    np.testing.assert_array_equal(oracle.log_mel(z, 80), -1.5)  # log10(1e-10) = -10 -> (-10 + 4) / 4
    x = _audio(48000, seed=9).astype(np.float64)
    a, b = oracle.log_mel(x, 80), oracle.log_mel(10.0 * x, 80)
    # x10 amplitude is x100 power, +2 in log10 everywhere, +0.5 after the rescale; the clamp moves with the max
    np.testing.assert_allclose(b - a, 0.5, atol=1e-9)
    assert a.max() - a.min() <= 2.0 + 1e-12  # the clamp holds everything within 8 / 4 of the top
