"""The GELU the GEMM epilogues evaluate (gelu_erf in
whisper_audio_encoder_amd/csrc/common.h), checked on the CPU from the
constants as committed.

The kernels write gelu(z) = max(z, 0) - |z| Q(|z|) with Q(u) = Phi(-u), the
upper normal tail, and Q(u) = 2^p(u), p a degree-5 polynomial whose
coefficients sit in common.h as fmaf literals.  This test parses them and
replays the kernel's arithmetic: Horner steps as fp32 fused multiply-adds
(each product of two fp32 values is exact in fp64, so fp64 followed by one
rounding to fp32 is the fused result), exp2 correctly rounded to fp32.  It
checks the claims the kernel's comment makes: |error| <= 4.7e-7 against the
exact erf GELU over [-12, 12], and p decreasing for all u >= 0, so the tail
term keeps shrinking past the fitted range.  tests/gelu_tail_fit.py derives
the coefficients; here they must also agree with a fresh fit.
"""
import os
import re

import numpy as np
from numpy.polynomial import polynomial as P
from scipy.special import erf

from tests import gelu_tail_fit

COMMON_H = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "whisper_audio_encoder_amd", "csrc", "common.h")


def committed_coefficients():
    """p's coefficients, constant term first, as the kernel's Horner chain has them."""
    src = open(COMMON_H).read()
    body = src[src.index("float gelu_erf(float z)"):]
    body = body[:body.index("exp2f")]
    lits = [np.float32(x) for x in re.findall(r"([-+]?\d\.\d+e[-+]\d+)f", body)]
    # fmaf(c5, u, c4), then fmaf(p, u, c3) ... fmaf(p, u, c0)
    assert len(lits) == 6, lits
    c5, c4, c3, c2, c1, c0 = lits
    return np.array([c0, c1, c2, c3, c4, c5], dtype=np.float32)


def fma32(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(np.float32)


def p32(c, u):
    """The kernel's Horner chain in fp32 fused multiply-adds."""
    acc = fma32(c[5], u, c[4])
    for k in (3, 2, 1, 0):
        acc = fma32(acc, u, c[k])
    return acc


def kernel_gelu(c, z):
    z = np.asarray(z, dtype=np.float32)
    u = np.abs(z)
    r = np.exp2(p32(c, u).astype(np.float64)).astype(np.float32)
    # fmaf(-u, r, max(z, 0)) in fp64, rounded once
    return (-u.astype(np.float64) * r + np.maximum(z, 0).astype(np.float64))


def exact_gelu(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))


def test_gelu_error_bound_over_the_range():
    c = committed_coefficients()
    z = np.linspace(-12.0, 12.0, 2_400_001).astype(np.float32)
    err = np.abs(kernel_gelu(c, z) - exact_gelu(z))
    assert err.max() <= 4.7e-7, err.max()
    # every fp16 input in [-16, 16] (what fc1's output rounding can see)
    h = np.arange(0, 65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h) & (np.abs(h) <= 16)]
    assert np.abs(kernel_gelu(c, h) - exact_gelu(h)).max() <= 4.7e-7


def test_tail_polynomial_decreases_for_all_u():
    c = committed_coefficients().astype(np.float64)
    d = P.polyder(c)
    # p'(u) < 0 on [0, inf): negative at 0 and no real root of p' >= 0 (the
    # leading coefficient is negative, so p' -> -inf)
    assert c[5] < 0 and P.polyval(0.0, d) < 0
    roots = P.polyroots(d)
    real = roots[np.abs(roots.imag) < 1e-12].real
    assert not np.any(real >= 0), real
    # and in the kernel's own fp32 arithmetic, on a wide grid
    u = np.linspace(0.0, 1e4, 1_000_001).astype(np.float32)
    assert np.all(np.diff(p32(committed_coefficients(), u)) <= 0)


def test_far_tail_underflows_to_relu():
    c = committed_coefficients()
    z = np.array([-1e4, -200.0, -40.0, 40.0, 200.0, 1e4], dtype=np.float32)
    g = kernel_gelu(c, z)
    assert np.array_equal(g, np.maximum(z, 0).astype(np.float64))


def test_coefficients_reproduce_from_the_fit():
    fresh = gelu_tail_fit.fit()
    np.testing.assert_allclose(fresh, committed_coefficients(), rtol=1e-5, atol=1e-7)
