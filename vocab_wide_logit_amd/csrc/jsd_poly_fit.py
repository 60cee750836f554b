"""Fits the small-argument polynomial of the JSD element term used by the
AsymSpec kernel (pass C) and prints its fp32 coefficients.

For one vocabulary element with log-probability difference x = ln p - ln q
(nats), rho = exp(-|x|) and Mx = max(p, q), the element's JSD contribution is
Mx * (1 + rho) / 2 * h(x) with the even function
    h(x) = x * tanh(x / 2) - 2 * ln cosh(x / 2).
The kernel accumulates Mx * g with g = -(1 + rho) * h(x) / (2 ln 2), so that
D = -(ln 2 / 2) * sum Mx * g.  For |x| < X0 it evaluates g = (1 + rho) * s * Q(s),
s = x^2, with Q(s) ~ -h(x) / (2 ln 2 x^2) fitted here by relative least squares
on Chebyshev nodes; for |x| >= X0 the closed form in rho and log2(1 + rho)
is accurate to a few 1e-7 relative.

    python jsd_poly_fit.py [X0] [degree]
"""
import sys

import numpy as np


def h_exact(x):
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    small = np.abs(x) < 0.02
    y = x[small] / 2
    out[small] = y ** 2 - y ** 4 / 2 + 2 * y ** 6 / 9
    xl = x[~small]
    out[~small] = xl * np.tanh(xl / 2) - 2 * np.log(np.cosh(xl / 2))
    return out


def fit(x0=1.2, deg=4, n=4000):
    k = np.arange(n)
    s = x0 ** 2 * 0.5 * (1 - np.cos(np.pi * (k + 0.5) / n))
    q = h_exact(np.sqrt(s)) / s
    A = np.vander(s, deg + 1, increasing=True)
    coef, *_ = np.linalg.lstsq(A / q[:, None], np.ones_like(q), rcond=None)
    return (-coef / (2 * np.log(2))).astype(np.float32)


def check(cf, x0):
    xs = np.linspace(1e-4, x0, 200001).astype(np.float32)
    s = (xs * xs).astype(np.float32)
    q = np.float32(cf[-1])
    for c in cf[-2::-1]:
        q = (q * s + c).astype(np.float32)
    val = (s * q).astype(np.float64)
    ex = -h_exact(xs.astype(np.float64)) / (2 * np.log(2))
    return float(np.max(np.abs(val / ex - 1)))


if __name__ == "__main__":
    x0 = float(sys.argv[1]) if len(sys.argv) > 1 else 1.2
    deg = int(sys.argv[2]) if len(sys.argv) > 2 else 4
    cf = fit(x0, deg)
    print("max relative error of the fp32 evaluation on (0, %g): %.3g" % (x0, check(cf, x0)))
    for i, c in enumerate(cf):
        print("constexpr float kJsdQ%d = %sf;" % (i, float.hex(float(c)).replace("0000000p", "p")))
