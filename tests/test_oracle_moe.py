"""Pins for the oracle's routed MoE FFN (CPU).

* the grouped (sorted-rows) forward equals a per-token brute-force loop
* E = k = 1 reduces to a dense SwiGLU FFN written out with explicit
  effective weights (formed only in this test)
* B = 0 per projection zeroes that projection's dA; experts with no rows get
  exactly zero adapter gradients
* finite differences of L = <dY, y> for x, router logits and every adapter
"""
import numpy as np
import pytest

import synth
from oracle import moe as om
from oracle import routing as orr
from oracle.blocks import act


def tiny(T=6, H=64, I=32, E=4, k=2, qtype=1, seed=0, large=True, zipf=0.0):
    cfg = synth.MoECfg("tiny", T=T, H=H, I=I, E=E, k=k, qtype=qtype, rank=2, alpha=4, zipf=zipf,
                       seed=seed)
    return synth.make_moe(cfg, large_adapter=large, w_sigma=0.1, threads=1)


@pytest.mark.parametrize("qtype", [0, 1, 2])
def test_grouped_equals_bruteforce(qtype):
    inp = tiny(T=12, E=6, k=2, qtype=qtype)
    f = om.forward(inp)
    _, _, yb = om.forward_bruteforce(inp)
    for t, v in yb.items():
        np.testing.assert_allclose(f["y"][t], v, rtol=1e-12, atol=1e-12)


def test_single_expert_is_dense_swiglu():
    inp = tiny(T=5, E=1, k=1)
    ew = om.ExpertWeights(inp).get(0)
    Wg, Wu, Wd, Ag, Au, Bg, Bu, Ad, Bd = ew
    s = float(inp["scale"])
    x = act(inp["x"])
    g = x @ (Wg + s * Bg @ Ag).T
    u = x @ (Wu + s * Bu @ Au).T
    y = ((g / (1 + np.exp(-g))) * u) @ (Wd + s * Bd @ Ad).T
    f = om.forward(inp)
    np.testing.assert_allclose(f["w"], 1.0)
    np.testing.assert_allclose(f["y"], y, rtol=1e-12, atol=1e-12)


def test_zero_b_and_idle_experts():
    inp = tiny(T=8, E=8, k=1)
    # route every token to experts 0..3 only
    lg = np.full((8, 8), -5.0, np.float32)
    for t in range(8):
        lg[t, t % 4] = 1.0
    inp["logits"] = lg
    inp["bg"][:] = 0.0
    f = om.forward(inp)
    b = om.backward(inp, f)
    assert np.all(b["dAg"] == 0.0)
    assert np.abs(b["dBg"][:4]).sum() > 0
    for n in ("dAg", "dAu", "dBg", "dBu", "dAd", "dBd"):
        assert np.all(b[n][4:] == 0.0), n


def test_finite_differences():
    inp = tiny(T=4, H=64, I=32, E=4, k=2)
    # well-separated logits so a small perturbation cannot change the top-k set
    lg = np.array([[2.0, 1.0, -1.0, -2.0], [-2.0, 1.5, 0.5, -1.0],
                   [0.3, -2.0, 1.2, -0.8], [-1.0, -0.5, 0.9, 2.2]])
    inp["logits"] = lg
    inp["x"] = act(inp["x"])
    inp["dy"] = act(inp["dy"])
    for n in ("ag", "au", "bg", "bu", "ad", "bd"):
        inp[n] = inp[n].astype(np.float64)
    f = om.forward(inp)
    b = om.backward(inp, f)

    def L():
        return float((inp["dy"] * om.forward(inp, keep=False)["y"]).sum())

    rng = np.random.default_rng(1)
    h = 1e-5

    def check(arr, grad, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = L()
        arr[idx] = old - h
        lm = L()
        arr[idx] = old
        fd = (lp - lm) / (2 * h)
        assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (idx, fd, grad[idx])

    for _ in range(6):
        check(inp["x"], b["dx"], (rng.integers(4), rng.integers(64)))
    for t in range(4):
        for e in range(4):
            check(inp["logits"], b["dlogits"], (t, e))
    for name, gname in (("ag", "dAg"), ("au", "dAu"), ("bg", "dBg"), ("bu", "dBu"),
                        ("ad", "dAd"), ("bd", "dBd")):
        arr, grad = inp[name], b[gname]
        for _ in range(4):
            idx = tuple(int(rng.integers(s)) for s in arr.shape)
            check(arr, grad, idx)


def test_expert_rows_helper_matches_full_backward():
    inp = tiny(T=10, E=5, k=2, qtype=2)
    f = om.forward(inp)
    b = om.backward(inp, f)
    ew = om.ExpertWeights(inp)
    for e in range(5):
        p0, p1 = f["offsets"][e], f["offsets"][e + 1]
        if p1 == p0:
            continue
        a = f["sorted"][p0:p1]
        r = om.expert_backward_rows(inp, e, a, f["w"].ravel()[a], ew)
        for n in ("dAg", "dAu", "dBg", "dBu", "dAd", "dBd"):
            np.testing.assert_allclose(r[n], b[n][e], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r["dw"], b["dw"].ravel()[a], rtol=1e-12, atol=1e-14)


def test_zipf_bias_skews_load():
    cfg = synth.MoECfg("z", T=512, H=64, I=32, E=32, k=4, qtype=2, rank=2, alpha=4, zipf=1.0)
    rng = np.random.default_rng([0, 0])
    logits = rng.standard_normal((512, 32), dtype=np.float32)
    bias = synth.zipf_bias(32, 1.0, rng)
    ids, _ = orr.topk(logits + bias, 4)
    counts = np.bincount(ids.ravel(), minlength=32)
    heavy = np.argmin(-bias)  # rank 1
    assert counts[heavy] == counts.max()
    assert counts.max() > 4 * np.median(counts)


def test_spill_cases_have_spill_experts():
    """The GPU cases meant for the spill launches route at least one expert a
    remainder of 1..32 rows past its full 64-row tiles and at least one expert
    a full tile; one of them does the same for 128-row tiles, and one routes
    experts of 1..8 rows in all beside experts with full 128-row tiles (the
    backward spill; host-side routing check)."""
    from moe_cases import SPILL_CASES

    seen128 = seen_nn = False
    for T, H, I, E, k, qtype, r, zipf in SPILL_CASES:
        cfg = synth.MoECfg("t", T=T, H=H, I=I, E=E, k=k, qtype=qtype, rank=r, alpha=2.0 * r, zipf=zipf,
                           seed=T + E)
        rng = np.random.default_rng([cfg.seed, 0])
        logits = synth._normal(rng, (T, E), 1.0)
        if zipf:
            logits = (logits + synth.zipf_bias(E, zipf, rng)[None, :]).astype(np.float32)
        cnt = np.diff(orr.route(logits, k)[3])
        rem = cnt % 64
        assert np.any((rem >= 1) & (rem <= 32)) and np.any(cnt >= 64), (T, E)
        seen128 = seen128 or (np.any((cnt % 128 >= 1) & (cnt % 128 <= 32)) and np.any(cnt >= 128))
        seen_nn = seen_nn or (np.any((cnt >= 1) & (cnt <= 8)) and np.any(cnt >= 128))
    assert seen128 and seen_nn
