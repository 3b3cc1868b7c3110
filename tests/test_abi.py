"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side argument checks work without a GPU (no compute calls here)."""
import ctypes
import os
import subprocess

import pytest
import torch

from whisper_audio_encoder_amd import synth, wenc
from whisper_audio_encoder_amd.configs import CONFIGS

pytestmark = pytest.mark.skipif(not os.path.exists(wenc.LIB_PATH), reason="libwenc.so not built")


def test_exports_every_declared_symbol():
    L = wenc.lib()
    names = wenc.header_functions()
    assert {"wenc_create", "wenc_load", "wenc_forward", "wenc_destroy", "wenc_weights_nbytes",
            "wenc_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", wenc.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_hip_imports_resolve_in_torch_runtime():
    """Every HIP entry the library imports exists in the runtime torch loads,
    so the library can share torch's streams and device pointers."""
    torch_hip = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    und = subprocess.run(["nm", "-D", "--undefined-only", wenc.LIB_PATH], capture_output=True, text=True).stdout
    need = {l.split()[-1].split("@")[0] for l in und.splitlines() if l.split()[-1].startswith(("hip", "__hip"))}
    have = subprocess.run(["nm", "-D", "--defined-only", torch_hip], capture_output=True, text=True).stdout
    have = {l.split()[-1].split("@")[0] for l in have.splitlines()}
    assert need and need <= have, sorted(need - have)


def test_weights_nbytes_matches_blob():
    for name, cfg in CONFIGS.items():
        assert wenc.wenc_weights_nbytes(wenc.make_config(cfg)) == synth.weights_nbytes(cfg), name


@pytest.mark.parametrize("field,value", [
    ("head_dim", 32), ("d_model", 100), ("n_mels", 81), ("d_ff", 1534), ("n_layer", -1),
    ("n_frames", 3001), ("n_ctx", 0), ("ln_eps", 0.0), ("final_ln", 2), ("max_batch", 0),
    ("max_batch", 6000),
])
def test_invalid_config_rejected(field, value):
    c = wenc.make_config(CONFIGS["c1"])
    setattr(c, field, value)
    assert wenc.wenc_weights_nbytes(c) == 0
    h = ctypes.c_void_p(123)
    rc = wenc.lib().wenc_create(ctypes.byref(c), ctypes.byref(h))
    assert rc == wenc.WENC_EINVAL and h.value is None
    assert "wenc_create" in wenc.wenc_last_error()


def test_null_handles():
    L = wenc.lib()
    L.wenc_destroy(None)
    assert L.wenc_load(None, None, 0) == wenc.WENC_EINVAL
    assert L.wenc_forward(None, None, 1, None, None) == wenc.WENC_EINVAL
    assert L.wenc_forward_tap(None, None, 1, 0, None, None) == wenc.WENC_EINVAL
    assert L.wenc_forward_ctx(None, None, 1, 500, None, None) == wenc.WENC_EINVAL
    assert L.wenc_load_cross(None, 1, None, 0) == wenc.WENC_EINVAL
    assert L.wenc_prepare_cross(None, None, 1, 1500, None, None, None) == wenc.WENC_EINVAL
    assert L.wenc_profile(None, 0) == wenc.WENC_EINVAL
    assert L.wenc_create(None, None) == wenc.WENC_EINVAL
    assert wenc.wenc_last_error(None) != ""


def test_kernel_entry_argument_checks():
    L = wenc.lib()
    a = wenc.wenc_gemm_args()
    a.A = a.W = a.bias = a.C = 16
    a.M, a.N, a.K, a.lda, a.ldw, a.ldc = 10, 16, 12, 12, 12, 16  # K not a multiple of 8
    a.a_rows_per_batch = a.c_rows_per_batch = 10
    assert L.wenc_k_gemm(ctypes.byref(a), None) == wenc.WENC_EINVAL
    assert "multiples of 8" in wenc.wenc_last_error()
    a.K = a.lda = a.ldw = 16
    a.epilogue = 9
    assert L.wenc_k_gemm(ctypes.byref(a), None) == wenc.WENC_EINVAL
    a.epilogue = wenc.WENC_EPI_QKV
    a.q = a.k = a.vt = 16
    a.n_head, a.T = 1, 10  # N must be 192
    assert L.wenc_k_gemm(ctypes.byref(a), None) == wenc.WENC_EINVAL
    assert L.wenc_k_layernorm(None, None, None, None, 4, 6, 1e-5, 0, None) == wenc.WENC_EINVAL
    assert L.wenc_k_layernorm(None, None, None, None, 4, 4096, 1e-5, 0, None) == wenc.WENC_EINVAL
    assert L.wenc_k_attention(None, None, None, None, 1, 1, 10, 9, None) == wenc.WENC_EINVAL


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a HIP device is present")
def test_create_without_device_reports_enodev():
    c = wenc.make_config(CONFIGS["c0"])
    h = ctypes.c_void_p()
    assert wenc.lib().wenc_create(ctypes.byref(c), ctypes.byref(h)) == wenc.WENC_ENODEV
    assert "no HIP device" in wenc.wenc_last_error()


def test_cross_blob_size():
    """Per decoder layer: x_wk [d][d], x_wv [d][d], x_bv [d] in fp16."""
    for name, n in (("c0", 1), ("c4", 32)):
        cfg = CONFIGS[name]
        d = cfg.d_model
        want = 2 * n * (2 * d * d + d)
        assert wenc.wenc_cross_nbytes(wenc.make_config(cfg), n) == want
        assert synth.pack_cross_blob(cfg, synth.make_cross_params(cfg, n), n).nbytes == want
    assert wenc.wenc_cross_nbytes(wenc.make_config(CONFIGS["c0"]), 0) == 0
