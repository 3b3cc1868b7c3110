"""Shortened-context windows (drafts) on the GPU: wenc_forward_ctx through
the C ABI against the fp64 oracle.

A draft encodes the audio plus 5 s, at least 10 s, instead of 30 s (whisper
README, section Serving), i.e. 2 T' mel frames with T' >= 500 of the
1500 positions.  The inputs are the leading 2 T' frames of each workload's
seeded mel, encoded by the full model (the same weight blob).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, check_encoder_tolerance, dev, host, say
from tests.test_gpu_encoder import encoder, inputs
from whisper_audio_encoder_amd import wenc
from whisper_audio_encoder_amd.configs import CONFIGS

pytestmark = pytest.mark.gpu


def _draft_oracle(name, item, Td):
    cfg, mel, params, _ = inputs(name)
    return oracle.encode(mel[item, :2 * Td], params, cfg.n_layer, cfg.n_head, cfg.ln_eps, bool(cfg.final_ln))


def _draft(name, Td, batch=None, enc=None):
    cfg, mel, _, _ = inputs(name)
    m = np.ascontiguousarray(mel[:batch, :2 * Td])
    out = (enc or encoder(name)).forward(dev(m), n_ctx=Td)
    return host(out)


@functools.lru_cache(maxsize=None)
def _draft_batch(name, Td):
    cfg = inputs(name)[0]
    say(f"draft {name} n_ctx {Td} batch {cfg.batch}")
    out = _draft(name, Td)
    assert out.shape == (cfg.batch, Td, cfg.d_model)
    return out


# every window of each workload: 10 s drafts (the shortest the pages allow),
# and 15.54 s at c2 (a ragged tail in every tile dimension)
DRAFTS = [("c1", 500), ("c2", 777), ("c3", 500), ("c4", 500)]
CASES = [(n, Td, i) for n, Td in DRAFTS for i in range(CONFIGS[n].batch)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,Td,item", CASES, ids=[f"{n}-T{Td}-w{i}" for n, Td, i in CASES])
def test_draft_matches_oracle(name, Td, item):
    out = _draft_batch(name, Td)
    check_encoder_tolerance(out[item], _draft_oracle(name, item, Td), f"draft {name} T'={Td} window {item}")


@pytest.mark.parametrize("Td", [1, 2, 63, 64, 65, 250])
def test_draft_short_contexts_c0(Td):
    say(f"draft c0 n_ctx {Td}")
    out = _draft("c0", Td)
    check_encoder_tolerance(out[0], _draft_oracle("c0", 0, Td), f"draft c0 T'={Td}")


def test_full_context_is_forward():
    name = "c2"
    cfg, mel, _, _ = inputs(name)
    say("draft at the full context equals wenc_forward")
    full = host(encoder(name).forward(dev(mel)))
    assert np.array_equal(_draft(name, cfg.n_ctx), full)


def test_draft_packs_more_windows_per_chunk():
    """max_batch 2 holds 6 windows at T' = 500: batch 8 runs as 6 + 2 and must
    equal the single-chunk result of a handle with max_batch 8, bit for bit."""
    name = "c2"
    cfg, _, _, blob = inputs(name)
    say("draft chunking c2 max_batch 2, n_ctx 500")
    small = wenc.Encoder(cfg, blob, max_batch=2)
    try:
        chunked = _draft(name, 500, enc=small)
    finally:
        small.close()
    assert np.array_equal(chunked, _draft(name, 500))


def test_draft_argument_errors():
    cfg, mel, _, _ = inputs("c0")
    say("draft argument errors")
    h = encoder("c0").h
    m = dev(np.ascontiguousarray(mel[:, :1000]))
    out = torch.empty((1, 500, cfg.d_model), device=DEV)
    for bad in (0, -3, cfg.n_ctx + 1):
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_forward_ctx(h, m, 1, bad, out)
        assert e.value.code == wenc.WENC_EINVAL and "n_ctx" in str(e.value)
    wenc.wenc_forward_ctx(h, m, 0, 500, out)  # empty batch: a no-op
