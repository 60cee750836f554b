"""Fits the polynomial of the one-exponential JSD element term used by the
AsymSpec divergence pass and prints its fp32 coefficients.

For one vocabulary element with probabilities p, q and x = ln p - ln q, the
element's share of D = JSD(P || Q) (natural log) is
    (p ln(2p/(p+q)) + q ln(2q/(p+q))) / 2 = sqrt(p q) * Psi(x) / 2,
    Psi(x) = cosh(x/2) * (x tanh(x/2) - 2 ln cosh(x/2)),
because (p + q)/2 = sqrt(p q) cosh(x/2) and, with tau = tanh(x/2),
(1+tau) ln(1+tau) + (1-tau) ln(1-tau) = x tanh(x/2) - 2 ln cosh(x/2).
Psi is even and analytic (its nearest singularities are at x = +-i*pi), so
with u = (x / X1)^2 in [0, 1] the kernel evaluates
    Psi(x) / 2 = u * P(u),   P of degree `deg`,
by Horner in fp32; sqrt(p q) is one exp2 of the mean log2-probability.
Elements with |x| >= X1 (and NaN or infinite x) are left to the exact
closed form.  P is fitted here for minimal maximum relative error (Lawson's
iteratively reweighted least squares on Chebyshev nodes).

    python jsd_psi_fit.py [X1] [degree]
"""
import sys

import numpy as np


def psi_half(x):
    """Psi(x)/2 in float64 (series below |x| = 0.02, where the closed form
    cancels)."""
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    small = np.abs(x) < 0.02
    y = x[small] / 2
    h_small = y ** 2 - y ** 4 / 2 + 2 * y ** 6 / 9           # h(x) = x tanh(x/2) - 2 ln cosh(x/2)
    out[small] = np.cosh(y) * h_small / 2
    xl = x[~small]
    h = xl * np.tanh(xl / 2) - 2 * np.log(np.cosh(xl / 2))
    out[~small] = np.cosh(xl / 2) * h / 2
    return out


def fit(x1=3.0, deg=6, n=6000, iters=80):
    k = np.arange(n)
    u = 0.5 * (1 - np.cos(np.pi * (k + 0.5) / n))
    f = psi_half(x1 * np.sqrt(u)) / u
    A = np.vander(u, deg + 1, increasing=True)
    w = np.ones_like(u)
    for _ in range(iters):
        sw = np.sqrt(w) / f
        c, *_ = np.linalg.lstsq(A * sw[:, None], f * sw, rcond=None)
        e = np.abs(A @ c - f) / f
        w = w * e
        w /= w.sum()
    return c.astype(np.float32)


def check(cf, x1):
    """Largest relative error of the fp32 Horner evaluation of u * P(u)."""
    xs = np.linspace(1e-4, x1, 400001)
    u = ((xs.astype(np.float32) * np.float32(1.0 / x1)) ** 2).astype(np.float32)
    acc = np.float32(cf[-1])
    for c in cf[-2::-1]:
        acc = (acc * u + c).astype(np.float32)
    val = (acc * u).astype(np.float64)
    ex = psi_half(x1 * np.sqrt(u.astype(np.float64)))
    return float(np.max(np.abs(val / ex - 1)))


if __name__ == "__main__":
    x1 = float(sys.argv[1]) if len(sys.argv) > 1 else 3.0
    deg = int(sys.argv[2]) if len(sys.argv) > 2 else 6
    cf = fit(x1, deg)
    print("max relative error of the fp32 evaluation on (0, %g): %.3g" % (x1, check(cf, x1)))
    for i, c in enumerate(cf):
        print("constexpr float kPsiP%d = %sf;" % (i, float.hex(float(c))))
