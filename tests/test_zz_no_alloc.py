"""The allocation-free greedy argmax (wenc_argmax_noalloc) through the C ABI
against the handle's wenc_argmax, bit for bit, and against the oracle.

Its chunk keys live in a device array the library's code object holds
(1 MiB per device) instead of a handle's scratch.  Two calls in a row, the
second smaller, check that a call's result does not depend on what an
earlier call left in the shared array; the large case runs in two passes
over the array.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, host, say
from whisper_audio_encoder_amd import synth, wenc
from whisper_audio_encoder_amd.configs import CONFIGS

pytestmark = pytest.mark.gpu

V = 51865  # Whisper's vocabulary


def _handle_argmax(enc, x):
    return host(enc.argmax(x)).astype(np.int64)


def _noalloc(x, rows=None, n=None):
    rows = x.shape[0] if rows is None else rows
    n = x.shape[1] if n is None else n
    out = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    wenc.wenc_argmax_noalloc(x, rows, n, x.stride(0), out)
    return host(out).astype(np.int64)


@pytest.fixture(scope="module")
def enc():
    cfg = CONFIGS["c0"]
    mel, params = synth.make_inputs(cfg)
    e = wenc.Encoder(cfg, synth.pack_blob(cfg, params))
    yield e
    e.close()


def test_noalloc_matches_handle_argmax_two_calls(enc):
    rng = np.random.default_rng(11)
    # first call: 6000 rows of the vocabulary (two passes over the array),
    # ties across chunk boundaries and NaNs planted
    big = (4 * rng.standard_normal((6000, V))).astype(np.float32)
    big[0, [2047, 2048]] = 40.0
    big[5999, [V - 2, V - 1]] = 40.0
    big[3000, 777] = np.nan
    # second call: fewer rows and a shorter row, so its chunk keys cover only
    # a prefix of what the first call wrote
    small = (4 * rng.standard_normal((9, 5000))).astype(np.float32)
    small[4, [100, 4097]] = 30.0
    for what, x in (("6000 x 51865", big), ("9 x 5000", small)):
        say(f"argmax_noalloc {what}")
        xd = torch.from_numpy(x).to(DEV)
        got = _noalloc(xd)
        np.testing.assert_array_equal(got, _handle_argmax(enc, xd), err_msg=what)
        np.testing.assert_array_equal(got, oracle.greedy_argmax(x), err_msg=what)


def test_noalloc_strided_rows_and_single_chunk():
    rng = np.random.default_rng(12)
    x = (4 * rng.standard_normal((16, V + 35))).astype(np.float32)
    say("argmax_noalloc strided rows")
    xd = torch.from_numpy(x).to(DEV)
    got = _noalloc(xd, 16, V)
    np.testing.assert_array_equal(got, oracle.greedy_argmax(x[:, :V]))
    one = (4 * rng.standard_normal((3, 2048))).astype(np.float32)  # one chunk: no keys at all
    np.testing.assert_array_equal(_noalloc(torch.from_numpy(one).to(DEV)), oracle.greedy_argmax(one))


def test_noalloc_allocates_nothing():
    """Free device memory (as the runtime reports it) does not change across a
    call, and torch's allocator sees no new block."""
    rng = np.random.default_rng(13)
    xd = torch.from_numpy((4 * rng.standard_normal((16, V))).astype(np.float32)).to(DEV)
    out = torch.empty((16,), dtype=torch.int32, device=DEV)
    wenc.wenc_argmax_noalloc(xd, 16, V, V, out)  # first call on the device looks the array up
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        wenc.wenc_argmax_noalloc(xd, 16, V, V, out)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0 and torch.cuda.memory_allocated() == alloc0


def test_noalloc_error_paths():
    say("argmax_noalloc errors")
    x = torch.zeros((2, 64), device=DEV)
    out = torch.empty((2,), dtype=torch.int32, device=DEV)
    for args in ((x, 2, 0, 64, out), (x, 2, 65, 64, out), (x, -1, 64, 64, out)):
        with pytest.raises(wenc.WencError) as e:
            wenc.wenc_argmax_noalloc(*args)
        assert e.value.code == wenc.WENC_EINVAL
    # beyond the static array: 131073 chunk keys per row
    with pytest.raises(wenc.WencError) as e:
        wenc.wenc_argmax_noalloc(x, 1, 131073 * 2048, 131073 * 2048, out)
    assert e.value.code == wenc.WENC_EINVAL and "static scratch" in str(e.value)
    raw = torch.zeros(64 * 4 + 2, dtype=torch.uint8, device=DEV)
    with pytest.raises(wenc.WencError) as e:
        wenc.wenc_argmax_noalloc(raw[2:], 1, 64, 64, out)
    assert e.value.code == wenc.WENC_EINVAL and "aligned" in str(e.value)
    wenc.wenc_argmax_noalloc(x, 0, 64, 64, out)  # no rows: a no-op
