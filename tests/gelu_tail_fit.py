"""How the coefficients of the kernels' GELU (gelu_erf in
whisper_audio_encoder_amd/csrc/common.h) were derived.

gelu(z) = z Phi(z) = max(z, 0) - |z| Q(|z|), where Q(u) = Phi(-u) is the
upper tail of the standard normal distribution.  The kernel evaluates
Q(u) = 2^p(u) with p a degree-5 polynomial in u; fit() fits p to log2 Q on
[0, 6] by iteratively reweighted least squares that drives down the largest
absolute error of u Q(u) (the error the GELU inherits) and rounds the
coefficients to fp32.  tests/test_gelu_constants.py checks the committed
coefficients (parsed from common.h) against the exact GELU and for
monotonicity; this script reproduces them:
    python tests/gelu_tail_fit.py
"""
import numpy as np
from numpy.polynomial import polynomial as P
from scipy.special import erf, erfc

DEG, U_MAX = 5, 6.0


def tail(u):
    return 0.5 * erfc(u / np.sqrt(2.0))


def fit():
    u = np.linspace(0.0, U_MAX, 40001)
    target = np.log2(tail(u))
    w = np.ones_like(u)
    best = None
    for _ in range(200):
        c = P.polyfit(u, target, DEG, w=w)
        err = np.abs(u * np.exp2(P.polyval(u, c)) - u * tail(u))
        if best is None or err.max() < best[0]:
            best = (err.max(), c.copy())
        w = w * (1.0 + 3.0 * err / err.max())
        w /= w.max()
    return best[1].astype(np.float32)


def horner32(c, u):
    acc = np.full_like(u, c[-1])
    for k in range(len(c) - 2, -1, -1):
        acc = (acc * u + c[k]).astype(np.float32)
    return acc


def main():
    c = fit()
    z = np.linspace(-12.0, 12.0, 2400001).astype(np.float32)
    u = np.abs(z)
    g = np.maximum(z, 0).astype(np.float64) - u * np.exp2(horner32(c, u).astype(np.float64))
    exact = 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))
    far = np.linspace(0.0, 1e4, 1000001).astype(np.float32)
    monotone = bool(np.all(np.diff(horner32(c, far)) <= 0))
    print("coefficients, constant term first:", ", ".join(f"{x:.9e}" for x in c))
    print(f"max |gelu error| on [-12, 12]: {np.abs(g - exact).max():.2e}; p decreasing on [0, 1e4]: {monotone}")


if __name__ == "__main__":
    main()
