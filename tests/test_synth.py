"""The seeded generator: determinism, sizes and distributions."""
import numpy as np
import pytest

from whisper_audio_encoder_amd import synth
from whisper_audio_encoder_amd.configs import CONFIGS


def test_param_counts():
    # encoder parameter counts of the five workloads (millions)
    expect = {"c0": 2.89, "c1": 8.21, "c2": 20.59, "c3": 88.15, "c4": 636.97}
    for name, m in expect.items():
        n = synth.weights_nbytes(CONFIGS[name]) // 2
        assert abs(n / 1e6 - m) < 0.01, name


def test_blob_deterministic_and_sized():
    cfg = CONFIGS["c1"]
    mel_a, pa = synth.make_inputs(cfg)
    mel_b, pb = synth.make_inputs(cfg)
    ba, bb = synth.pack_blob(cfg, pa), synth.pack_blob(cfg, pb)
    assert ba.nbytes == synth.weights_nbytes(cfg)
    assert np.array_equal(ba, bb) and np.array_equal(mel_a, mel_b)
    mel_c, pc = synth.make_inputs(cfg, seed=cfg.seed + 1)
    assert not np.array_equal(mel_a, mel_c)


def test_distributions():
    cfg = CONFIGS["c2"]
    mel, params = synth.make_inputs(cfg)
    assert mel.dtype == np.float32 and mel.shape == (8, 3000, 80)
    assert mel.min() >= -1.5 and mel.max() <= 1.5
    assert abs(mel.mean() + 0.2) < 0.01 and abs(mel.std() - 0.4) < 0.01
    w = params["l0.fc1_w"].astype(np.float64)
    assert abs(w.std() - 0.02) < 5e-4 and abs(w.mean()) < 5e-4
    g = params["l3.ln2_g"].astype(np.float64)
    assert abs(g.mean() - 1.0) < 5e-3
    assert all(v.dtype == np.float16 for v in params.values())
    # independent batch items: no two windows equal
    assert not np.array_equal(mel[0], mel[1])


def test_position_table():
    pos = synth.sinusoid_table(1500, 512)
    # row 0 is sin(0)=0 then cos(0)=1; every entry lies in [-1, 1]
    assert np.all(pos[0, :256] == 0) and np.all(pos[0, 256:] == 1)
    assert np.abs(pos).max() <= 1.0
    # the first column pair rotates at one radian per frame (omega_0 = 1)
    t = np.arange(1500)
    np.testing.assert_allclose(pos[:, 0], np.sin(t), atol=1e-12)
    # the last frequency is 1/10000 rad per frame
    np.testing.assert_allclose(pos[:, 255], np.sin(t * 1e-4), atol=1e-12)


def test_pack_rejects_wrong_dtype():
    cfg = CONFIGS["c0"]
    _, params = synth.make_inputs(cfg)
    params["conv1_b"] = params["conv1_b"].astype(np.float32)
    with pytest.raises(ValueError):
        synth.pack_blob(cfg, params)
