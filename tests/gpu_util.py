"""Helpers shared by the GPU tests: device tensors, comparison metrics."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    """Name the case about to run on the GPU (flushed, so a fault still shows it)."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def f16_dev(a):
    return dev(np.asarray(a, dtype=np.float16))


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def row_cosine(got, ref):
    got = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = (got * ref).sum(1)
    den = np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1)
    return num / np.maximum(den, 1e-300)


def check_encoder_tolerance(got, ref, what=""):
    """The end-to-end bar: per-row cosine >= 0.9999 and max |err| <= 3e-2."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    cos = row_cosine(got, ref).min()
    err = np.abs(got - ref).max()
    say(f"{what}: min row cosine {cos:.7f}, max abs err {err:.3e}")
    assert cos >= 0.9999, f"{what}: min row cosine {cos}"
    assert err <= 3e-2, f"{what}: max abs err {err}"
    return cos, err
