"""Pins for the oracle's fused linear layer and its fast LoRA backward (CPU).

* closed forms: B = 0 (base only, dA = 0), A = 0 (dB = 0), s = 0, identity
  weight (y = x exactly), one-hot rows pick a column of deq(W)
* finite differences of L = <dY, y> in x, A and B (L is linear in x and
  bilinear in (A, B), so central differences are exact up to rounding)
* agreement with an explicit W_eff = deq(W) + s B A (formed only here)
"""
import numpy as np
import pytest

import synth
from oracle import blocks as ob
from oracle import linear as ol


def _small(T=5, K=64, N=32, r=2, s=2.0, qtype=0, seed=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K))
    W = ob.dequant(qtype, synth.quantize(qtype, (0.1 * rng.standard_normal((N, K))).astype(np.float32)), N, K)
    A = rng.standard_normal((r, K)) * 0.3
    B = rng.standard_normal((N, r)) * 0.3
    dy = rng.standard_normal((T, N))
    return x, W, A, B, dy, s


def test_b_zero_gives_base_only():
    x, W, A, B, dy, s = _small()
    B0 = np.zeros_like(B)
    y, _ = ol.forward(x, W, A, B0, s)
    assert np.array_equal(y, x @ W.T)
    dx, dA, dB = ol.backward(x, dy, W, A, B0, s)
    assert np.all(dA == 0.0)
    assert np.abs(dB).sum() > 0


def test_a_zero_gives_zero_db():
    x, W, A, B, dy, s = _small()
    _, _, dB = ol.backward(x, dy, W, np.zeros_like(A), B, s)
    assert np.all(dB == 0.0)


def test_scale_zero():
    x, W, A, B, dy, _ = _small()
    y, _ = ol.forward(x, W, A, B, 0.0)
    assert np.array_equal(y, x @ W.T)
    dx, dA, dB = ol.backward(x, dy, W, A, B, 0.0)
    assert np.array_equal(dx, dy @ W)
    assert np.all(dA == 0) and np.all(dB == 0)


def test_identity_weight_q8_0():
    K = 64
    raw = np.zeros((K, K // 32, 34), np.uint8)
    raw[..., 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    for n in range(K):
        raw[n, n // 32, 2 + n % 32] = 1
    W = ob.dequant(0, raw.reshape(K, -1), K, K)
    assert np.array_equal(W, np.eye(K))
    x = ob.bf16_value(synth.f32_to_bf16_bits(np.random.default_rng(0).standard_normal((3, K)).astype(np.float32)))
    y, _ = ol.forward(x, W, np.zeros((2, K)), np.zeros((K, 2)), 2.0)
    assert np.array_equal(y, x)


def test_one_hot_rows_select_columns():
    x, W, A, B, dy, s = _small(T=4, K=64, N=32)
    X = np.zeros((4, 64))
    cols = [0, 17, 33, 63]
    for t, c in enumerate(cols):
        X[t, c] = 1.0
    y, _ = ol.forward(X, W, A, np.zeros_like(B), s)
    for t, c in enumerate(cols):
        assert np.array_equal(y[t], W[:, c])


@pytest.mark.parametrize("T", [3, 5])
def test_finite_differences(T):
    x, W, A, B, dy, s = _small(T=T)
    dx, dA, dB = ol.backward(x, dy, W, A, B, s)

    def L(x_, A_, B_):
        return float((dy * ol.forward(x_, W, A_, B_, s)[0]).sum())

    h = 1e-3
    rng = np.random.default_rng(3)
    for _ in range(12):
        i, j = rng.integers(T), rng.integers(x.shape[1])
        e = np.zeros_like(x); e[i, j] = h
        fd = (L(x + e, A, B) - L(x - e, A, B)) / (2 * h)
        assert abs(fd - dx[i, j]) <= 1e-7 * max(1.0, abs(dx[i, j]))
        a, b = rng.integers(A.shape[0]), rng.integers(A.shape[1])
        e = np.zeros_like(A); e[a, b] = h
        fd = (L(x, A + e, B) - L(x, A - e, B)) / (2 * h)
        assert abs(fd - dA[a, b]) <= 1e-7 * max(1.0, abs(dA[a, b]))
        a, b = rng.integers(B.shape[0]), rng.integers(B.shape[1])
        e = np.zeros_like(B); e[a, b] = h
        fd = (L(x, A, B + e) - L(x, A, B - e)) / (2 * h)
        assert abs(fd - dB[a, b]) <= 1e-7 * max(1.0, abs(dB[a, b]))


def test_matches_explicit_effective_weight():
    x, W, A, B, dy, s = _small(T=7, K=128, N=96, r=4)
    Weff = W + s * B @ A
    y, _ = ol.forward(x, W, A, B, s)
    np.testing.assert_allclose(y, x @ Weff.T, rtol=1e-12, atol=1e-12)
    dx, _, _ = ol.backward(x, dy, W, A, B, s)
    np.testing.assert_allclose(dx, dy @ Weff, rtol=1e-12, atol=1e-12)


def test_run_on_synth_input():
    cfg = synth.LinearCfg("t", T=16, K=64, N=96, qtype=1, rank=4, alpha=8)
    inp = synth.make_linear(cfg)
    out = ol.run(inp)
    assert out["y"].shape == (16, 96) and out["dx"].shape == (16, 64)
    assert out["dA"].shape == (4, 64) and out["dB"].shape == (96, 4)
