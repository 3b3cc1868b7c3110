"""The log-mel kernel's filter tables (host logic, no GPU) against the
oracle's Slaney filter bank (oracle/frontend.py, pinned to HF's filter bank
and to closed forms in test_oracle_frontend.py).

wenc_log_mel reads filter m through a window of 16 nch bins from mstart[m]
(CKE page, "The Frontend": the triangles are sparse, so the kernel does not
multiply a dense 201-bin row).  Here: every window lies inside bins 0..200,
holds every non-zero weight of its triangle, those weights are the oracle's
rounded to fp32 (the host builds them in fp64), the rest of the window is
zero, and nch is the smallest that fits the widest triangle.
"""
import ctypes

import numpy as np
import pytest

import oracle.frontend as fe
from whisper_audio_encoder_amd import wenc


@pytest.mark.parametrize("n_mels", list(range(8, 129, 8)))
def test_windows_hold_the_oracle_filters(n_mels):
    mstart, mwt = wenc.wenc_k_logmel_tables(n_mels)
    width = mwt.shape[1]
    assert width % 16 == 0
    ref = fe.mel_filters(n_mels)  # fp64 [n_mels][201]
    assert np.all(mstart >= 0) and np.all(mstart + width <= 201)
    dense = np.zeros((n_mels, 201))
    for m in range(n_mels):
        dense[m, mstart[m]:mstart[m] + width] = mwt[m]
    # the oracle's weights to fp32 rounding; at a triangle's corner the two
    # fp64 evaluations of the corner frequency may leave ~1e-17 on one side
    # and an exact zero on the other, hence the tiny absolute slack
    np.testing.assert_allclose(dense, ref, rtol=2 ** -23, atol=1e-15)
    assert np.all(dense[ref > 1e-15] > 0)
    runs = [np.flatnonzero(r) for r in dense]
    widest = max(r[-1] - r[0] + 1 for r in runs if r.size)
    assert (width - 16) < widest <= width  # the fewest 16-bin windows that hold it


def test_whisper_banks_need_one_window():
    """80 and 128 filters: every triangle fits 16 bins (14 and 9 at most)."""
    for n_mels in (80, 128):
        assert wenc.wenc_k_logmel_tables(n_mels)[1].shape[1] == 16


def test_bad_arguments():
    for n_mels in (0, -3, 1, 7, 129, 136):
        with pytest.raises(ValueError):
            wenc.wenc_k_logmel_tables(n_mels)
    nch = ctypes.c_int32()
    ms = np.zeros(80, dtype=np.int32)
    mw = np.zeros(80 * 16, dtype=np.float32)
    L = wenc.lib()
    assert L.wenc_k_logmel_tables(80, None, None, None, 0) == wenc.WENC_EINVAL
    assert L.wenc_k_logmel_tables(80, ctypes.byref(nch), ms.ctypes.data, mw.ctypes.data, mw.size - 1) == wenc.WENC_EINVAL
    assert "mwt holds" in wenc.wenc_last_error()
    assert L.wenc_k_logmel_tables(80, ctypes.byref(nch), ms.ctypes.data, mw.ctypes.data, mw.size) == wenc.WENC_OK
