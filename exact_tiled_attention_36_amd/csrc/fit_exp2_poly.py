"""Coefficients of the software 2^f used by fa_fwd_variant 3 (see poly_exp2 in common.h).

2^x is split as 2^n * 2^f with n = rint(x), f = x - n in [-1/2, 1/2] (Cody-Waite style
argument reduction); 2^f is a degree-3 polynomial whose coefficients minimise the
largest relative error on [-1/2, 1/2], found by Lawson's iteratively reweighted least
squares on a dense grid. Run this file to reproduce them (and the error bound)."""
import numpy as np


def fit(deg: int = 3, iters: int = 200):
    f = np.linspace(-0.5, 0.5, 20001)
    y = np.exp2(f)
    V = np.vander(f, deg + 1, increasing=True)
    w = np.ones_like(f)
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(V * (w / y)[:, None], w, rcond=None)
        err = (V @ c - y) / y
        w = w * np.abs(err)
        w /= w.sum()
    c32 = c.astype(np.float32)
    p = np.full_like(f, c32[-1], dtype=np.float32)
    for k in range(deg - 1, -1, -1):
        p = p * f.astype(np.float32) + c32[k]
    return c32, float(np.max(np.abs(p.astype(np.float64) - y) / y))


if __name__ == "__main__":
    c, err = fit()
    print("coefficients c0..c3:", [float(x) for x in c])
    print("max relative error (float32 Horner):", err)
