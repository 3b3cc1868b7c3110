"""Decode-step cross-attention on the GPU (wenc_cross_attend through the C
ABI) against the fp64 oracle.

A generated token's query rows attend over the n_ctx encoder positions
through one decoder layer's cached K/V (whisper README, "Performance and
memory": one query per sequence, the keys split across blocks and the
partial softmaxes merged; whisper 0.9.0 API page, wh_prepare_cross).  The
oracle takes the exact fp16 values the kernel reads.

Tolerance from the arithmetic: the scores are exact fp16 products summed in
fp32, the probabilities and sums stay fp32, and the output is rounded to
fp16 once: rtol 1e-3, atol 1e-4 (one fp16 rounding, 2^-11 relative).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, dev, f16_dev, host, say
from tests.test_gpu_cross import _loaded
from tests.test_gpu_encoder import encoder, inputs
from whisper_audio_encoder_amd import wenc

pytestmark = pytest.mark.gpu


def _case(rng, B, H, n_q, T, q_scale=1.0, dominant=False):
    d = 64 * H
    q = (q_scale * rng.standard_normal((B, n_q, d))).astype(np.float16)
    xk = rng.standard_normal((B, T, d)).astype(np.float16)
    xv = rng.standard_normal((B, T, d)).astype(np.float16)
    if dominant:  # one key per (item, head) aligned with query 0: a +60-ish score margin
        for b in range(B):
            for h in range(H):
                u = int(rng.integers(0, T))
                c = slice(64 * h, 64 * h + 64)
                xk[b, u, c] = (np.sign(q[b, 0, c].astype(np.float32)) * 4).astype(np.float16)
    return q, xk, xv


def _oracle(q, xk, xv, H):
    return np.stack([oracle.cross_attend(q[b], xk[b], xv[b], H) for b in range(q.shape[0])])


def _run(enc, q, xk, xv):
    out = enc.cross_attend(f16_dev(q), f16_dev(xk), f16_dev(xv))
    return host(out).astype(np.float64)


# (config whose handle is used, B, n_q, T).  The first eleven take the
# two-pass path: 16 windows x 20 heads at one query row and 1500 keys (the
# decode step the benchmark times: more pairs than compute units); then few
# (b, h) pairs: one query at the full 1500 keys; a few queries;
# beams of 8; ragged key counts against the keys a workgroup of the first
# pass takes (512 for up to 4 query rows, 256 for more): one key, 64, 257,
# 513 (one workgroup + 1), 777, 1024 (exactly two) and 257 with 6 rows.  The
# next four take the one-pass path on a 256-CU MI355X (up to 4 rows and
# B x n_head pairs of 0.7 to 1.0 per CU): full, ragged and single keys (T = 1
# leaves every wave but the first without a tile).  The last three are large
# batches of 5 to 8 rows, which keep the two passes.
CASES = [("c4", 16, 1, 1500), ("c4", 2, 1, 1500), ("c4", 3, 3, 777), ("c3", 2, 8, 1500), ("c3", 4, 2, 257),
         ("c1", 1, 1, 1), ("c1", 5, 4, 64), ("c2", 8, 1, 1500), ("c3", 3, 2, 513), ("c2", 2, 4, 1024),
         ("c1", 3, 6, 257),
         ("c4", 12, 1, 1500), ("c3", 16, 3, 777), ("c2", 24, 2, 513), ("c1", 40, 4, 1),
         ("c4", 8, 8, 1500), ("c2", 40, 6, 65), ("c1", 30, 5, 777)]


@pytest.mark.parametrize("name,B,n_q,T", CASES)
def test_cross_attend_matches_oracle(name, B, n_q, T):
    cfg = inputs(name)[0]
    H = cfg.n_head
    say(f"cross attend {name} B={B} H={H} n_q={n_q} T={T}")
    rng = np.random.default_rng(B * 1000 + n_q * 100 + T)
    q, xk, xv = _case(rng, B, H, n_q, T)
    got = _run(encoder(name), q, xk, xv)
    np.testing.assert_allclose(got, _oracle(q, xk, xv, H), rtol=1e-3, atol=1e-4)


@pytest.mark.parametrize("q_scale,dominant", [(8.0, False), (1.0, True)])
def test_cross_attend_sharp_scores(q_scale, dominant):
    """Peaked softmaxes: scores with a standard deviation of 8, and one key per
    head with a margin of tens (the partial maxima differ widely between
    key chunks, so the merge's rescaling matters)."""
    H, B, n_q, T = 20, 2, 2, 1500
    say(f"cross attend sharp q_scale={q_scale} dominant={dominant}")
    rng = np.random.default_rng(int(q_scale) * 7 + dominant)
    q, xk, xv = _case(rng, B, H, n_q, T, q_scale=q_scale, dominant=dominant)
    got = _run(encoder("c4"), q, xk, xv)
    np.testing.assert_allclose(got, _oracle(q, xk, xv, H), rtol=1e-3, atol=1e-4)


def test_cross_attend_on_prepared_cross_kv():
    """The decoder path end to end at whisper-tiny shapes: the library's own
    encoder memory, its cached K/V for every decoder layer, then one query
    row per window and layer; the oracle takes the cached fp16 K/V."""
    cfg, _, enc = _loaded("c1")
    _, mel, _, _ = inputs("c1")
    memory = enc.forward(dev(mel))
    xk, xv = enc.prepare_cross(memory)
    rng = np.random.default_rng(5)
    say(f"cross attend on prepared K/V c1: {xk.shape[0]} layers")
    for layer in range(xk.shape[0]):
        q = rng.standard_normal((cfg.batch, 1, cfg.d_model)).astype(np.float16)
        got = host(enc.cross_attend(f16_dev(q), xk[layer].contiguous(), xv[layer].contiguous())).astype(np.float64)
        ref = _oracle(q, host(xk[layer]), host(xv[layer]), cfg.n_head)
        np.testing.assert_allclose(got, ref, rtol=1e-3, atol=1e-4)


def test_cross_attend_deterministic_and_chunked():
    """Bit-identical repeats; a batch larger than the handle's scratch holds
    at once (c0's handle, one window of scratch) is processed in chunks with
    the same bits as item-by-item calls."""
    cfg = inputs("c0")[0]
    H, B, n_q, T = cfg.n_head, 40, 8, 1500
    say(f"cross attend chunking B={B} n_q={n_q} T={T}")
    rng = np.random.default_rng(11)
    q, xk, xv = _case(rng, B, H, n_q, T)
    enc = encoder("c0")
    qd, kd, vd = f16_dev(q), f16_dev(xk), f16_dev(xv)
    a = host(enc.cross_attend(qd, kd, vd))
    b = host(enc.cross_attend(qd, kd, vd))
    assert np.array_equal(a, b)
    for i in (0, 17, 39):
        one = host(enc.cross_attend(qd[i:i + 1].contiguous(), kd[i:i + 1].contiguous(), vd[i:i + 1].contiguous()))
        assert np.array_equal(one[0], a[i])
    np.testing.assert_allclose(a[[0, 39]].astype(np.float64), _oracle(q[[0, 39]], xk[[0, 39]], xv[[0, 39]], H),
                               rtol=1e-3, atol=1e-4)


@pytest.mark.parametrize("name,B,n_q,T", [("c4", 12, 1, 1500), ("c3", 16, 4, 700), ("c2", 30, 3, 1500),
                                           ("c1", 40, 2, 1)])
def test_cross_attend_one_pass_matches_two_passes_bitwise(name, B, n_q, T):
    """A batch whose (b, h) pairs about fill a 256-CU MI355X once runs the
    one-pass kernel; each of its items alone runs the two launches.  The one
    pass repeats the two passes' arithmetic in their order, so every output
    bit agrees: the result does not depend on the batch it was computed in."""
    H = inputs(name)[0].n_head
    say(f"cross attend one pass vs two {name} B={B} n_q={n_q} T={T}")
    rng = np.random.default_rng(B * 31 + n_q * 7 + T)
    q, xk, xv = _case(rng, B, H, n_q, T, q_scale=4.0)
    enc = encoder(name)
    qd, kd, vd = f16_dev(q), f16_dev(xk), f16_dev(xv)
    a = host(enc.cross_attend(qd, kd, vd))
    for i in sorted({0, B // 2, B - 1}):
        one = host(enc.cross_attend(qd[i:i + 1].contiguous(), kd[i:i + 1].contiguous(), vd[i:i + 1].contiguous()))
        assert np.array_equal(one[0].view(np.uint16), a[i].view(np.uint16)), f"item {i}"
    np.testing.assert_allclose(a[[0, B - 1]].astype(np.float64), _oracle(q[[0, B - 1]], xk[[0, B - 1]],
                               xv[[0, B - 1]], H), rtol=1e-3, atol=1e-4)


def test_cross_attend_error_paths():
    enc = encoder("c1")
    L = wenc.lib()
    d = enc.cfg.d_model
    q = torch.zeros((1, 1, d), dtype=torch.float16, device=DEV)
    kv = torch.zeros((1, 10, d), dtype=torch.float16, device=DEV)
    p = lambda t: t.data_ptr()  # noqa: E731
    assert L.wenc_cross_attend(enc.h, p(q), p(kv), p(kv), 1, 0, 10, p(q), None) == wenc.WENC_EINVAL
    assert L.wenc_cross_attend(enc.h, p(q), p(kv), p(kv), 1, 9, 10, p(q), None) == wenc.WENC_EINVAL
    assert L.wenc_cross_attend(enc.h, p(q), p(kv), p(kv), 1, 1, 0, p(q), None) == wenc.WENC_EINVAL
    assert L.wenc_cross_attend(enc.h, p(q), p(kv), p(kv), 1, 1, enc.cfg.n_ctx + 1, p(q), None) == wenc.WENC_EINVAL
    assert L.wenc_cross_attend(enc.h, p(q), None, p(kv), 1, 1, 10, p(q), None) == wenc.WENC_EINVAL
    assert L.wenc_cross_attend(enc.h, p(q) + 2, p(kv), p(kv), 1, 1, 10, p(q), None) == wenc.WENC_EINVAL
    assert L.wenc_cross_attend(enc.h, p(q), p(kv), p(kv), -1, 1, 10, p(q), None) == wenc.WENC_EINVAL
    assert L.wenc_cross_attend(None, p(q), p(kv), p(kv), 1, 1, 10, p(q), None) == wenc.WENC_EINVAL
    assert L.wenc_cross_attend(enc.h, None, None, None, 0, 1, 10, None, None) == wenc.WENC_OK
