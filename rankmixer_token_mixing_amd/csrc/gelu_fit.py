"""Coefficients of the GELU used by the HIP kernels (common.hpp, gelu_erf).

GELU(x) = x Phi(x) = max(x, 0) - |x| Phi(-|x|), Phi the standard normal CDF.
The kernels evaluate the tail as
    Phi(-a) = exp2(P(min(a, 6.5))),
with P a degree-6 polynomial fitted here to log2 Phi(-a) on [0, 6.5] by
least squares weighted by the size of the tail term a Phi(-a).  The
Gaussian's -log2(e) a^2 / 2 is a polynomial term of P, so it costs no
separate operations; beyond the clamp the tail stays at Phi(-6.5) ~ 4e-11,
an error of |x| * 4e-11 in GELU(x).  Run to print the
coefficients (highest power first) and the float32 error of the kernel's
formula against the exact GELU.  Needs numpy and scipy; used at development
time only, nothing imports it.
"""
import numpy as np
from scipy.special import erf, log_ndtr

A = 6.5
DEG = 6
L2E = 1.0 / np.log(2.0)


def fit():
    a = np.linspace(0.0, A, 400001)
    g = log_ndtr(-a) * L2E
    w = np.sqrt(np.maximum(a * np.exp(log_ndtr(-a)), 1e-12))
    V = np.vander(a, DEG + 1)
    c, *_ = np.linalg.lstsq(V * w[:, None], g * w, rcond=None)
    return c.astype(np.float32)


def gelu_f32(x, c):
    f = np.float32
    ax = np.abs(x)
    ac = np.minimum(ax, f(A))
    p = np.full_like(ac, c[0])
    for ck in c[1:]:
        p = p * ac + ck
    e = np.exp2(p).astype(f)
    return np.maximum(x, f(0)) - ax * e


if __name__ == "__main__":
    c = fit()
    print("coefficients:", ", ".join(f"{float(v)!r}f" for v in c))
    x = np.linspace(-9, 9, 3000001).astype(np.float32)
    xd = x.astype(np.float64)
    ref = 0.5 * xd * (1 + erf(xd / np.sqrt(2)))
    err = np.abs(gelu_f32(x, c) - ref)
    m = np.abs(ref) > 1e-3
    print(f"max abs error {err.max():.2e}, max rel error where |GELU| > 1e-3: {(err[m] / np.abs(ref[m])).max():.2e}")
