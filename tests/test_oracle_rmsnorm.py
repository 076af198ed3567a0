"""Pins for the oracle's RMS normalisation (CPU).

* closed forms: a constant row c gives y = w * c / sqrt(c^2 + eps); a row
  scaled by a > 0 gives the same y when eps = 0; mean((y / w)^2) over a row
  equals mean(x^2) / (mean(x^2) + eps)
* brute force: rstd from a per-element Python loop on a tiny input
* the backward: central finite differences of L = <dY, y>; with eps = 0,
  y is invariant to scaling x, so every row of dx is orthogonal to x
"""
import math

import numpy as np

from oracle import rmsnorm as orms


def test_constant_row_closed_form():
    H, c, eps = 16, -0.75, 1e-3
    x = np.full((1, H), c)
    w = np.linspace(0.5, 2.0, H)
    y, rstd = orms.forward(x, w, eps)
    assert math.isclose(rstd[0], 1.0 / math.sqrt(c * c + eps), rel_tol=1e-15)
    np.testing.assert_allclose(y[0], w * c / math.sqrt(c * c + eps), rtol=1e-15)


def test_scale_invariance_without_eps():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 40))
    w = rng.standard_normal(40)
    y1, _ = orms.forward(x, w, 0.0)
    y2, _ = orms.forward(7.5 * x, w, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-15)


def test_mean_square_of_normalised_rows():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 24)) * 3.0
    w = rng.uniform(0.5, 1.5, 24)
    eps = 0.25
    y, _ = orms.forward(x, w, eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean((y / w) ** 2, axis=1), ms / (ms + eps), rtol=1e-13)


def test_rstd_brute_force():
    x = np.array([[1.0, -2.0, 3.0, 0.5], [0.0, 0.0, 0.0, 2.0]])
    w = np.ones(4)
    eps = 1e-2
    _, rstd = orms.forward(x, w, eps)
    for t in range(2):
        s = 0.0
        for v in x[t]:
            s += v * v
        assert math.isclose(rstd[t], 1.0 / math.sqrt(s / 4 + eps), rel_tol=1e-15)


def test_backward_finite_differences():
    rng = np.random.default_rng(5)
    T, H, eps = 3, 12, 0.1
    x = rng.standard_normal((T, H))
    w = rng.standard_normal(H)
    dy = rng.standard_normal((T, H))
    dx = orms.backward(x, w, dy, eps)
    h = 1e-6
    num = np.zeros_like(x)
    for t in range(T):
        for j in range(H):
            xp, xm = x.copy(), x.copy()
            xp[t, j] += h
            xm[t, j] -= h
            num[t, j] = (np.sum(dy * orms.forward(xp, w, eps)[0]) -
                         np.sum(dy * orms.forward(xm, w, eps)[0])) / (2 * h)
    np.testing.assert_allclose(dx, num, rtol=1e-7, atol=1e-9)


def test_backward_orthogonal_to_x_without_eps():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 32))
    w = rng.standard_normal(32)
    dy = rng.standard_normal((5, 32))
    dx = orms.backward(x, w, dy, 0.0)
    np.testing.assert_allclose(np.sum(dx * x, axis=1), 0.0, atol=1e-12)
