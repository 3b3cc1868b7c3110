"""Greedy argmax of a decode step on the GPU (wenc_argmax through the C ABI)
against the oracle, bit for bit.

The index is an integer decided by comparisons alone (no arithmetic), so
the two sides must agree exactly, ties, signed zeros, infinities and NaNs
included (whisper README, "Performance and memory": the argmax over the
51865 logits is reduced on the device and one integer comes back).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, host, say
from tests.test_gpu_encoder import encoder
from whisper_audio_encoder_amd import wenc

pytestmark = pytest.mark.gpu

V = 51865  # Whisper's vocabulary


def _logits(rng, rows, n):
    return (4 * rng.standard_normal((rows, n))).astype(np.float32)


def _run(x, enc=None):
    enc = enc or encoder("c1")
    got = enc.argmax(torch.from_numpy(np.ascontiguousarray(x)).to(DEV))
    return host(got).astype(np.int64)


# (rows, n_vocab): the decode shape; one row; one chunk exactly, one logit
# past it, a ragged tail; a single logit; many short rows
SHAPES = [(16, V), (1, V), (5, 2048), (5, 2049), (7, 777), (3, 1), (300, 130), (2, 4096 * 3 + 5)]


@pytest.mark.parametrize("rows,n", SHAPES)
def test_argmax_matches_oracle(rows, n):
    say(f"argmax rows={rows} n={n}")
    rng = np.random.default_rng(rows * 7 + n)
    x = _logits(rng, rows, n)
    np.testing.assert_array_equal(_run(x), oracle.greedy_argmax(x))


def test_argmax_ties_zeros_infinities_nans():
    """Maxima tied across chunk boundaries (2047 | 2048, 4095 | 4096) and in
    the ragged last chunk, signed zeros, rows of -inf, +inf ties, NaNs early
    and late, adjacent fp32 values, subnormals."""
    rng = np.random.default_rng(3)
    x = _logits(rng, 14, V)
    x[0, [2047, 2048, 4096]] = 50.0
    x[1, [4095, 4096]] = 50.0
    x[2, [V - 1, V - 2]] = 50.0
    x[3] = -1.0
    x[3, [9000, 100]] = [-0.0, 0.0]
    x[4] = -np.inf
    x[5, [30000, 20000, 40000]] = np.inf
    x[6, 51000] = np.nan
    x[7, [3, 2]] = [np.nan, np.inf]
    x[8, V - 1] = np.nan
    x[9, 777] = 40.0
    x[9, 30000] = np.nextafter(np.float32(40.0), np.float32(41.0))
    x[10] = 0.0
    x[10, [5, 6]] = [-1e-45, 1e-45]
    x[11] = -0.0
    x[12] = np.float32(3.4e38)
    x[13] = -np.float32(3.4e38)
    x[13, 12345] = -np.float32(3.3e38)
    want = oracle.greedy_argmax(x)
    np.testing.assert_array_equal(_run(x), want)
    assert list(want[:12]) == [2047, 4095, V - 2, 100, 0, 20000, 51000, 3, V - 1, 30000, 6, 0]


def test_argmax_strided_rows():
    """Rows of a wider buffer (ld = n_vocab + 3, so rows start off any
    16-byte boundary)."""
    rng = np.random.default_rng(4)
    full = _logits(rng, 9, V + 3)
    want = oracle.greedy_argmax(full[:, :V])
    d = torch.from_numpy(full).to(DEV)
    got = host(encoder("c1").argmax(d[:, :V])).astype(np.int64)
    np.testing.assert_array_equal(got, want)


def test_argmax_chunked_by_scratch_and_deterministic():
    """6000 rows of 51865 logits on whisper-tiny's one-window handle, whose
    scratch holds the chunk keys of 5538 rows: two passes.  Sampled rows
    (both sides of the pass boundary, the ends, planted ties) against the
    oracle; every row equal to a handle whose scratch takes them in one pass; repeats
    bit-identical."""
    rows = 6000
    g = torch.Generator(device=DEV).manual_seed(7)
    say(f"argmax chunked rows={rows} n={V}")
    d = 4 * torch.randn((rows, V), device=DEV, generator=g)
    d[5538, [10, 11, 2048]] = 60.0
    d[5537, V - 1] = float("nan")
    small = encoder("c0")
    a = host(small.argmax(d)).astype(np.int64)
    b = host(small.argmax(d)).astype(np.int64)
    assert np.array_equal(a, b)
    big = host(encoder("c1", max_batch=64).argmax(d)).astype(np.int64)
    assert np.array_equal(a, big)
    rng = np.random.default_rng(8)
    sample = sorted({0, 1, 5536, 5537, 5538, 5539, rows - 1, *rng.integers(0, rows, 12).tolist()})
    want = oracle.greedy_argmax(host(d[sample]))
    np.testing.assert_array_equal(a[sample], want)
    assert a[5538] == 10 and a[5537] == V - 1
    del d


def test_argmax_error_paths():
    enc = encoder("c1")
    L = wenc.lib()
    x = torch.zeros((2, 64), dtype=torch.float32, device=DEV)
    o = torch.zeros((2,), dtype=torch.int32, device=DEV)
    p = lambda t: t.data_ptr()  # noqa: E731
    assert L.wenc_argmax(enc.h, p(x), -1, 64, 64, p(o), None) == wenc.WENC_EINVAL
    assert L.wenc_argmax(enc.h, p(x), 2, 0, 64, p(o), None) == wenc.WENC_EINVAL
    assert L.wenc_argmax(enc.h, p(x), 2, 64, 63, p(o), None) == wenc.WENC_EINVAL
    assert L.wenc_argmax(enc.h, p(x), 2, (1 << 30) + 1, 1 << 31, p(o), None) == wenc.WENC_EINVAL
    assert L.wenc_argmax(enc.h, None, 2, 64, 64, p(o), None) == wenc.WENC_EINVAL
    assert L.wenc_argmax(enc.h, p(x), 2, 64, 64, None, None) == wenc.WENC_EINVAL
    assert L.wenc_argmax(enc.h, p(x) + 2, 2, 64, 64, p(o), None) == wenc.WENC_EINVAL
    assert L.wenc_argmax(None, p(x), 2, 64, 64, p(o), None) == wenc.WENC_EINVAL
    assert L.wenc_argmax(enc.h, None, 0, 64, 64, None, None) == wenc.WENC_OK
    with pytest.raises(ValueError):
        enc.argmax(x.double())
    with pytest.raises(ValueError):
        enc.argmax(x.t())
