"""Pins for the oracle's LM head with chunked cross entropy (CPU).

* W = 0 and B = 0 give loss = ln V exactly and zero dh, dA
* the chunked online log-sum-exp equals the direct one; chunk size does not
  matter (4096-style chunks with a ragged tail, tiny chunks, one chunk)
* rows of G sum to zero, so sum_v dB[v, :] = 0
* finite differences of the loss in h, A and B
* ignored labels: zero rows; all ignored: zero loss and gradients
* statistical sanity: with iid logits of variance sigma^2 the mean loss is
  close to ln V + sigma^2 / 2
"""
import math

import numpy as np
import pytest

import synth
from oracle import lmhead as olm
from oracle.blocks import act


def tiny(T=3, H=32, V=50, chunk=16, qtype=0, seed=0, ignore_frac=0.0, large=True, w_sigma=0.1):
    cfg = synth.HeadCfg("tiny", T=T, H=H, V=V, qtype=qtype, rank=2, alpha=4, chunk=chunk,
                        ignore_frac=ignore_frac, seed=seed)
    return synth.make_head(cfg, large_adapter=large, w_sigma=w_sigma, threads=1)


def test_zero_weights_give_log_v():
    inp = tiny(T=4, V=151936 // 32, H=32)
    inp["blocks"][:] = 0  # d = 0 -> every weight 0
    inp["B"][:] = 0.0
    out = olm.forward_backward(inp)
    assert abs(out["loss"] - math.log(inp["V"])) < 1e-12
    assert np.all(out["dh"] == 0.0) and np.all(out["dA"] == 0.0)


@pytest.mark.parametrize("chunk", [16, 7, 50, 4096])
def test_chunked_equals_direct(chunk):
    inp = tiny(T=5, V=50, chunk=chunk, qtype=1)
    d = olm.forward_backward_direct(inp)
    c = olm.forward_backward(inp, chunk=chunk)
    assert abs(c["loss"] - d["loss"]) < 1e-12
    for n in ("lse", "dh", "dA", "dB"):
        np.testing.assert_allclose(c[n], d[n], rtol=1e-11, atol=1e-14)


def test_db_columns_sum_to_zero():
    inp = tiny(T=6, V=64, qtype=2)
    out = olm.forward_backward(inp)
    assert np.abs(out["dB"].sum(axis=0)).max() < 1e-14
    assert np.abs(out["dB"]).max() > 1e-6


def test_finite_differences():
    inp = tiny(T=3, H=32, V=50, chunk=16)
    inp["h"] = act(inp["h"])
    inp["A"] = inp["A"].astype(np.float64)
    inp["B"] = inp["B"].astype(np.float64)
    out = olm.forward_backward(inp)
    rng = np.random.default_rng(2)
    h = 1e-6

    def check(arr, grad, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = olm.forward_backward(inp, want_grad=False)["loss"]
        arr[idx] = old - h
        lm = olm.forward_backward(inp, want_grad=False)["loss"]
        arr[idx] = old
        fd = (lp - lm) / (2 * h)
        assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(grad[idx])), (idx, fd, grad[idx])

    for _ in range(10):
        check(inp["h"], out["dh"], (rng.integers(3), rng.integers(32)))
        check(inp["A"], out["dA"], (rng.integers(2), rng.integers(32)))
        check(inp["B"], out["dB"], (rng.integers(50), rng.integers(2)))


def test_ignore_index():
    inp = tiny(T=8, V=40, chunk=16)
    inp["labels"][[1, 4]] = -100
    out = olm.forward_backward(inp)
    assert out["n_valid"] == 6
    assert np.all(out["dh"][[1, 4]] == 0.0)
    keep = [0, 2, 3, 5, 6, 7]
    sub = dict(inp, h=inp["h"][keep], labels=inp["labels"][keep], T=6)
    ref = olm.forward_backward(sub)
    assert abs(ref["loss"] - out["loss"]) < 1e-12
    np.testing.assert_allclose(out["dh"][keep], ref["dh"], rtol=1e-12, atol=1e-15)
    inp["labels"][:] = -100
    out = olm.forward_backward(inp)
    assert out["loss"] == 0.0 and np.all(out["dh"] == 0) and np.all(out["dB"] == 0)


def test_statistical_sanity():
    inp = tiny(T=1024, H=256, V=4096, chunk=1024, qtype=0, large=False, w_sigma=0.02)
    out = olm.forward_backward(inp, want_grad=False)
    sigma2 = 256 * 0.02 ** 2
    # label-logit noise has sd sqrt(sigma2 / T) = 0.01; allow 4 sd
    assert abs(out["loss"] - (math.log(4096) + sigma2 / 2)) < 0.04


def test_two_class_softplus():
    """V = 2, h = e_0, W rows (3, 0, ...) and (-1, 0, ...) give logits (3, -1):
    loss = ln(1 + e^(z_other - z_label)), a closed form for each label."""
    inp = tiny(T=2, H=32, V=2, chunk=16)
    raw = np.zeros((2, 34), np.uint8)
    raw[:, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    raw[0, 2] = 3
    raw[1, 2] = np.uint8(np.int8(-1).view(np.uint8))
    inp["blocks"] = raw
    inp["B"][:] = 0.0
    h = np.zeros((2, 32)); h[:, 0] = 1.0
    inp["h"] = h
    inp["labels"] = np.array([0, 1])
    out = olm.forward_backward(inp)
    want = (math.log1p(math.exp(-4.0)) + math.log1p(math.exp(4.0))) / 2
    assert abs(out["loss"] - want) < 1e-14
    np.testing.assert_allclose(out["lse"], [math.log(math.exp(3) + math.exp(-1))] * 2, rtol=1e-15)
