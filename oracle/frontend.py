"""Plain fp64 definition of Whisper's log-mel frontend.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import or call this module.

Source: CKE page ("How Audio Becomes Words"), section "The Frontend: Sound
Becomes A Tensor": a fixed 30-s window of 480,000 samples at 16 kHz; STFT
power with n_fft 400, hop 160, a periodic Hann window and reflect padding,
giving 201 frequency bins by 3000 frames; n_mels triangular filters on the
Slaney mel scale, area-normalised (80, or 128 for large-v3: section "Tiny,
Base, Small, Large"); log10; a clamp at 8 below the largest value of the
whole window (-80 dB); and the (x + 4) / 4 rescale.  The same page checks
this chain against Hugging Face's WhisperFeatureExtractor.

Readings where the pages are silent (recorded in the design notes): frames
are centred (frame t starts at sample 160 t - 200 of the reflect-padded
signal) and the STFT's last frame is dropped, which is how 480,000 samples
give exactly 3000 frames; the filters span 0 Hz to the Nyquist frequency
8 kHz; power is floored at 1e-10 before log10 (log10 of a silent bin would
otherwise be -inf, and the clamp needs a finite maximum); the output is
frame-major [n_frames][n_mels], the layout the encoder reads.

Library steps: numpy's FFT (the pages name numpy.fft as their FFT check) and
elementwise numpy; no blocking, no reduced precision.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
SAMPLE_RATE = 16000
N_FFT = 400
HOP = 160


def hann_periodic(n: int = N_FFT) -> np.ndarray:
    """w[j] = 0.5 - 0.5 cos(2 pi j / n), j < n (periodic: the DFT-even window)."""
    j = np.arange(n, dtype=F64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * j / n)


def stft_power(audio, n_frames: int | None = None) -> np.ndarray:
    """|STFT|^2 of one window: [n_frames][N_FFT // 2 + 1] in fp64.

    audio: [n_samples] with n_samples = HOP * n_frames.  Frame t covers
    samples 160 t - 200 .. 160 t + 199, read from the signal reflected about
    its first and last samples (the edge sample itself is not repeated);
    X[t][k] = sum_j w[j] x[160 t - 200 + j] exp(-2 pi i j k / 400).
    """
    x = np.asarray(audio, dtype=F64)
    n = x.shape[0]
    if n_frames is None:
        n_frames = n // HOP
    half = N_FFT // 2
    xp = np.pad(x, (half, half), mode="reflect")
    idx = HOP * np.arange(n_frames)[:, None] + np.arange(N_FFT)[None, :]
    frames = xp[idx] * hann_periodic()[None, :]
    spec = np.fft.rfft(frames, axis=1)
    return spec.real ** 2 + spec.imag ** 2


def hz_to_mel_slaney(f):
    """Slaney's auditory-toolbox scale: linear (200/3 Hz per mel) below
    1 kHz, logarithmic above (27 mels per factor 6.4)."""
    f = np.asarray(f, dtype=F64)
    lin = f / (200.0 / 3.0)
    logpart = 15.0 + np.log(np.maximum(f, 1e-300) / 1000.0) / (np.log(6.4) / 27.0)
    return np.where(f >= 1000.0, logpart, lin)


def mel_to_hz_slaney(m):
    m = np.asarray(m, dtype=F64)
    lin = m * (200.0 / 3.0)
    logpart = 1000.0 * np.exp((np.log(6.4) / 27.0) * (m - 15.0))
    return np.where(m >= 15.0, logpart, lin)


def mel_filters(n_mels: int, n_fft: int = N_FFT, sr: int = SAMPLE_RATE) -> np.ndarray:
    """[n_mels][n_fft // 2 + 1] triangular filters.

    Filter i rises linearly from corner f_i to f_{i+1} and falls to f_{i+2},
    the n_mels + 2 corners evenly spaced in Slaney mels from 0 Hz to sr / 2;
    bin k sits at k sr / n_fft Hz.  Area normalisation scales filter i by
    2 / (f_{i+2} - f_i), which gives the continuous triangle unit area.
    """
    bins = np.arange(n_fft // 2 + 1, dtype=F64) * sr / n_fft
    corners = mel_to_hz_slaney(np.linspace(0.0, hz_to_mel_slaney(sr / 2.0), n_mels + 2))
    fb = np.zeros((n_mels, bins.size), dtype=F64)
    for i in range(n_mels):
        lo, mid, hi = corners[i], corners[i + 1], corners[i + 2]
        rise = (bins - lo) / (mid - lo)
        fall = (hi - bins) / (hi - mid)
        fb[i] = np.maximum(0.0, np.minimum(rise, fall)) * (2.0 / (hi - lo))
    return fb


def log_mel(audio, n_mels: int, n_frames: int | None = None) -> np.ndarray:
    """Whisper's log-mel of one window: [n_frames][n_mels] in fp64."""
    p = stft_power(audio, n_frames)
    m = p @ mel_filters(n_mels).T
    lg = np.log10(np.maximum(m, 1e-10))
    lg = np.maximum(lg, lg.max() - 8.0)
    return (lg + 4.0) / 4.0
