"""Pins for the oracle's 8-bit AdamW (CPU).

* code books: 256 values, strictly increasing with the magnitude code, top
  value 1, one group of codes per decade, spot values worked out by hand
* quantize: every book value maps back to its own code; the chosen code is
  the nearest by brute force over the whole book
* a step worked out by hand (two elements, exact binary fractions): the new
  p, the codes chosen for both states, the block scales
* with states the books hold exactly, the oracle's update equals the
  library AdamW of PyTorch (torch.optim.AdamW in float64) step for step
* the first step from zero states is plain sign descent up to eps
* a block whose scale is below the smallest normal float32 stores code 0
  while a normal block beside it does not
* several quantised steps stay within the quantisation error of the
  unquantised library AdamW
"""
import numpy as np
import torch

from oracle import adamw8bit as oa


def test_code_books():
    tu, ts = oa.unsigned_table(), oa.signed_table()
    assert tu.shape == (256,) and ts.shape == (256,)
    assert tu[0] == 0 and tu[255] == 1.0
    assert np.all(np.diff(tu) > 0)
    assert np.all(np.diff(ts[:128]) > 0) and ts[127] == 1.0
    np.testing.assert_array_equal(ts[128:], -ts[:128])
    # by hand: unsigned code 1 (e = 7, no fraction bits): 1e-7 * (0.1 + 0.9);
    # code 2 = 0b10 (e = 6, f = 1, i = 0): 1e-6 * (0.1 + 0.45) = 5.5e-7;
    # code 3 = 0b11 (i = 1): 1e-6; code 255: 1
    np.testing.assert_allclose(tu[[1, 2, 3, 255]], [1e-7, 5.5e-7, 1e-6, 1.0], rtol=1e-15)
    # signed magnitude code 74 = 0b1001010 (e = 0, f = 6, i = 10):
    # 0.1 + 0.9 * 11 / 64 = 0.2546875; code 100 of the unsigned book =
    # 0b01100100 (e = 1, f = 6, i = 36): 0.1 * (0.1 + 0.9 * 37 / 64) = 0.06203125
    assert ts[74] == 0.2546875 and ts[128 + 74] == -0.2546875
    np.testing.assert_allclose(tu[100], 0.06203125, rtol=1e-15)
    # the top group (e = 0, 7 fraction bits): 128 codes spread over (0.1, 1]
    np.testing.assert_allclose(tu[128:], 0.1 + 0.9 * np.arange(1, 129) / 128, rtol=1e-15)


def test_quantize_round_trip_and_nearest():
    tu, ts = oa.unsigned_table(), oa.signed_table()
    np.testing.assert_array_equal(oa.quantize(tu, tu), np.arange(256))
    codes = oa.quantize(ts, ts)
    np.testing.assert_array_equal(codes[:128], np.arange(128))
    np.testing.assert_array_equal(codes[129:], np.arange(129, 256))  # -0 stores as +0
    rng = np.random.default_rng(0)
    for table, x in ((tu, rng.uniform(0, 1, 2000)), (ts, rng.uniform(-1, 1, 2000))):
        x = x * 10.0 ** -rng.integers(0, 7, x.size)
        q = oa.quantize(x, table)
        best = np.min(np.abs(x[:, None] - table[None, :]), axis=1)
        np.testing.assert_array_equal(np.abs(x - table[q]), best)
        lo, hi, dmid = oa.neighbours(x, table)
        assert np.all(table[lo] <= x) and np.all(table[hi] >= x)
        assert np.all((q == lo) | (q == hi))


def test_hand_worked_step():
    # p = [1, 1], g = [0.5, -2], zero states, t = 1, lr 0.5, b1 0.5, b2 0.75,
    # eps 0.25, no weight decay.  By hand:
    #   m' = 0.5 g = [0.25, -1];  v' = 0.25 g^2 = [0.0625, 1]
    #   m'/(1 - 0.5) = [0.5, -2];  v'/(1 - 0.75) = [0.25, 4], sqrt [0.5, 2]
    #   p' = 1 - 0.5 [0.5 / 0.75, -2 / 2.25] = [2/3, 13/9]
    #   scales: max |m'| = 1, max v' = 1
    #   m codes: -1 -> sign | 127 = 255; 0.25 lies between 0.240625 (i = 8)
    #     and 0.2546875 (i = 10, code 74), nearer the latter
    #   v codes: 1 -> 255; 0.0625 lies between 0.06203125 (code 100) and
    #     0.0634375 (code 101), nearer the former
    r = oa.step_exact(np.ones(2, np.float32), np.array([0.5, -2.0], np.float32), np.zeros(2, np.uint8),
                      np.zeros(2, np.uint8), np.zeros(1, np.float32), np.zeros(1, np.float32),
                      1, 0.5, 0.5, 0.75, 0.25, 0.0)
    np.testing.assert_allclose(r["p"], [2 / 3, 13 / 9], rtol=1e-15)
    np.testing.assert_array_equal(r["m"], [0.25, -1.0])
    np.testing.assert_array_equal(r["v"], [0.0625, 1.0])
    assert r["scale_m"].tolist() == [1.0] and r["scale_v"].tolist() == [1.0]
    p, mq, vq, sm, sv = oa.step(np.ones(2, np.float32), np.array([0.5, -2.0], np.float32),
                                np.zeros(2, np.uint8), np.zeros(2, np.uint8), np.zeros(1, np.float32),
                                np.zeros(1, np.float32), 1, 0.5, 0.5, 0.75, 0.25, 0.0)
    assert mq.tolist() == [74, 255] and vq.tolist() == [100, 255]
    assert p.tolist() == [np.float32(2 / 3), np.float32(13 / 9)]


def _torch_adamw(p, g, m, v, t, lr, b1, b2, eps, wd):
    """One step of the library AdamW (float64, CPU) from states m, v at
    step t - 1."""
    pt = torch.tensor(np.asarray(p, np.float64), requires_grad=True)
    opt = torch.optim.AdamW([pt], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    pt.grad = torch.tensor(np.asarray(g, np.float64))
    if t > 1:
        opt.state[pt] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                         "exp_avg": torch.tensor(np.asarray(m, np.float64)),
                         "exp_avg_sq": torch.tensor(np.asarray(v, np.float64))}
    opt.step()
    st = opt.state[pt]
    return pt.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


def _f32(x):
    return float(np.float32(x))


def test_update_equals_library_adamw():
    """Random stored states (whatever codes and scales) dequantise to exact
    values; from those the oracle's update must be the library's."""
    rng = np.random.default_rng(5)
    n = 600
    lr, b1, b2, eps, wd = _f32(1e-3), _f32(0.9), _f32(0.999), _f32(1e-8), _f32(0.01)
    for t in (1, 2, 7, 100):
        p = rng.standard_normal(n).astype(np.float32)
        g = rng.standard_normal(n).astype(np.float32)
        mq = rng.integers(0, 256, n).astype(np.uint8)
        vq = rng.integers(0, 256, n).astype(np.uint8)
        sm = rng.uniform(0.01, 1, 3).astype(np.float32)
        sv = rng.uniform(0.01, 1, 3).astype(np.float32)
        if t == 1:
            mq[:] = 0
            vq[:] = 0
        r = oa.step_exact(p, g, mq, vq, sm, sv, t, lr, b1, b2, eps, wd)
        pl, ml, vl = _torch_adamw(p, g, r["m_in"], r["v_in"], t, lr, b1, b2, eps, wd)
        np.testing.assert_allclose(r["p"], pl, rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(r["m"], ml, rtol=1e-14, atol=1e-300)
        np.testing.assert_allclose(r["v"], vl, rtol=1e-14, atol=1e-300)
        # the scales are the block maxima and the normalised states their ratio
        for b in range(3):
            sl = slice(256 * b, min(n, 256 * (b + 1)))
            assert r["scale_m"][b] == np.abs(r["m"][sl]).max() and r["scale_v"][b] == r["v"][sl].max()
            np.testing.assert_array_equal(r["mn"][sl], r["m"][sl] / r["scale_m"][b])


def test_constant_gradient_states_stay_exact():
    """Each block's gradient entries share one magnitude: m and v stay at
    +-scale and scale, which both books hold exactly (code values +-1), so
    the quantised chain is the library AdamW for every step."""
    rng = np.random.default_rng(6)
    n = 512
    mag = np.repeat(np.array([0.3, 2.0], np.float32), 256)
    sign = np.where(rng.integers(0, 2, n) > 0, 1.0, -1.0).astype(np.float32)
    g = mag * sign
    p = rng.standard_normal(n).astype(np.float32)
    mq, vq = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    sm, sv = np.zeros(2, np.float32), np.zeros(2, np.float32)
    lr, b1, b2, eps, wd = _f32(1e-2), _f32(0.5), _f32(0.75), _f32(1e-3), _f32(0.1)
    pl, ml, vl = p.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, 6):
        r = oa.step_exact(p, g, mq, vq, sm, sv, t, lr, b1, b2, eps, wd)
        p, mq, vq, sm, sv = oa.step(p, g, mq, vq, sm, sv, t, lr, b1, b2, eps, wd)
        pl, ml, vl = _torch_adamw(pl, g, ml, vl, t, lr, b1, b2, eps, wd)
        np.testing.assert_allclose(r["m"], ml, rtol=1e-6)  # states come back through float32 scales
        assert set(np.unique(mq)) <= {127, 255} and set(np.unique(vq)) == {255}
        np.testing.assert_allclose(p, pl, rtol=1e-6, atol=1e-7)
        pl = p.astype(np.float64)  # continue the library chain from the stored p
        ml = oa.dequantize(mq, sm, oa.signed_table(), n)
        vl = oa.dequantize(vq, sv, oa.unsigned_table(), n)


def test_first_step_is_sign_descent():
    rng = np.random.default_rng(1)
    n = 700  # three blocks, the last ragged
    p = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    z8 = np.zeros(n, np.uint8)
    zs = np.zeros(3, np.float32)
    lr, eps, wd = _f32(1e-3), _f32(1e-8), _f32(0.01)
    r = oa.step_exact(p, g, z8, z8, zs, zs, 1, lr, 0.9, 0.999, eps, wd)
    gd, pd = g.astype(np.float64), p.astype(np.float64)
    expect = pd - lr * (gd / (np.abs(gd) + eps) + wd * pd)
    np.testing.assert_allclose(r["p"], expect, rtol=1e-14)
    b1 = _f32(0.9)
    np.testing.assert_allclose(r["scale_m"], [np.abs((1 - b1) * gd[i:i + 256]).max() for i in (0, 256, 512)],
                               rtol=1e-15)


def test_steps_track_library_adamw():
    rng = np.random.default_rng(2)
    n = 1000
    p = rng.standard_normal(n).astype(np.float32)
    mq = np.zeros(n, np.uint8)
    vq = np.zeros(n, np.uint8)
    sm = np.zeros(4, np.float32)
    sv = np.zeros(4, np.float32)
    pl, ml, vl = p.astype(np.float64), np.zeros(n), np.zeros(n)
    lr = 1e-3
    for t in range(1, 6):
        g = rng.standard_normal(n).astype(np.float32)
        p, mq, vq, sm, sv = oa.step(p, g, mq, vq, sm, sv, t, lr, 0.9, 0.999, 1e-8, 0.0)
        pl, ml, vl = _torch_adamw(pl, g, ml, vl, t, _f32(lr), _f32(0.9), _f32(0.999), _f32(1e-8), 0.0)
    # each step moves p by at most lr / (1 - 0.9) in size; the 8-bit states
    # perturb the direction by a few per cent of that
    assert np.max(np.abs(p - pl)) < 0.1 * 5 * lr


def test_subnormal_scale_block_stores_zero_codes():
    rng = np.random.default_rng(3)
    n = 512
    g = rng.standard_normal(n).astype(np.float32)
    g[256:] *= np.float32(1e-20)  # v = (1 - b2) g^2 ~ 1e-43: below 2^-126
    z8 = np.zeros(n, np.uint8)
    zs = np.zeros(2, np.float32)
    p1, mq, vq, sm, sv = oa.step(np.zeros(n, np.float32), g, z8, z8, zs, zs, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert 0 < sv[1] < 2.0 ** -126 and sv[0] > 2.0 ** -126
    assert np.all(vq[256:] == 0) and np.count_nonzero(vq[:256]) > 200
    # m = 0.1 g ~ 1e-21 is normal: its block keeps non-zero codes
    assert sm[1] > 2.0 ** -126 and np.count_nonzero(mq[256:]) > 200
