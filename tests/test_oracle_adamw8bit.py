"""Pins for the oracle's 8-bit AdamW (CPU).

* code books: 256 values, strictly increasing with the magnitude code, top
  value 1, one group of codes per decade, spot values from the rule by hand
* quantize: every code value maps back to its own code; the chosen code is
  the nearest by brute force over the whole book
* the first step from zero states is plain sign descent up to eps:
  p - lr (g / (|g| + eps) + wd p), whatever the code books
* a block whose scale is below the smallest normal float32 stores code 0
  (its reciprocal would overflow) while a normal block beside it does not
* several steps stay within the quantisation error of a float64 AdamW with
  unquantised states
"""
import numpy as np

from oracle import adamw8bit as oa


def test_code_books():
    tu, ts = oa.unsigned_table(), oa.signed_table()
    assert tu.shape == (256,) and ts.shape == (256,)
    assert tu[0] == 0 and tu[255] == 1.0
    assert np.all(np.diff(tu.astype(np.float64)) > 0)
    assert np.all(np.diff(ts[:128].astype(np.float64)) > 0) and ts[127] == 1.0
    np.testing.assert_array_equal(ts[128:], -ts[:128])
    # unsigned code 1: e = 7, no fraction bits -> 1e-7; code 0b11: e = 6, i = 1 of 2 -> 1e-6
    assert tu[1] == np.float32(1e-7) and tu[3] == np.float32(1e-6)
    assert tu[2] == np.float32(1e-6 * (0.1 + 0.9 * 0.5))
    # the top group (e = 0, 7 fraction bits): 128 codes spread over (0.1, 1]
    np.testing.assert_allclose(tu[128:], 0.1 + 0.9 * np.arange(1, 129) / 128, rtol=1e-7)


def test_quantize_round_trip_and_nearest():
    tu, ts = oa.unsigned_table(), oa.signed_table()
    np.testing.assert_array_equal(oa.quantize(tu, tu), np.arange(256))
    codes = oa.quantize(ts, ts)
    np.testing.assert_array_equal(codes[:128], np.arange(128))
    np.testing.assert_array_equal(codes[129:], np.arange(129, 256))  # -0 stores as +0
    rng = np.random.default_rng(0)
    for table, x in ((tu, rng.uniform(0, 1, 2000)), (ts, rng.uniform(-1, 1, 2000))):
        x = (x * 10.0 ** -rng.integers(0, 7, x.size)).astype(np.float32)
        q = oa.quantize(x, table)
        best = np.min(np.abs(x[:, None] - table[None, :]), axis=1)
        np.testing.assert_array_equal(np.abs(x - table[q]), best)


def test_first_step_is_sign_descent():
    rng = np.random.default_rng(1)
    n = 700  # three blocks, the last ragged
    p = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    z8 = np.zeros(n, np.uint8)
    zs = np.zeros(3, np.float32)
    lr, eps, wd = 1e-3, 1e-8, 0.01
    p1, mq, vq, sm, sv = oa.step(p, g, z8, z8, zs, zs, 1, lr, 0.9, 0.999, eps, wd)
    expect = p.astype(np.float64) - lr * (g / (np.abs(g.astype(np.float64)) + eps) + wd * p)
    # float32 p takes two roundings at its own scale (p * kd, then the
    # subtraction), each within 2^-24 relative; the lr-sized term adds ~1e-9
    np.testing.assert_allclose(p1, expect, rtol=2.5e-7, atol=1e-9)
    np.testing.assert_allclose(sm, [np.abs(0.1 * g[i:i + 256]).max() for i in (0, 256, 512)], rtol=1e-6)


def test_steps_track_float64_adamw():
    rng = np.random.default_rng(2)
    n = 1000
    p = rng.standard_normal(n).astype(np.float32)
    mq = np.zeros(n, np.uint8)
    vq = np.zeros(n, np.uint8)
    sm = np.zeros(4, np.float32)
    sv = np.zeros(4, np.float32)
    p64, m64, v64 = p.astype(np.float64), np.zeros(n), np.zeros(n)
    lr = 1e-3
    for t in range(1, 6):
        g = rng.standard_normal(n).astype(np.float32)
        p, mq, vq, sm, sv = oa.step(p, g, mq, vq, sm, sv, t, lr, 0.9, 0.999, 1e-8, 0.0)
        p64, m64, v64 = oa.step_fp64(p64, g, m64, v64, t, lr, 0.9, 0.999, 1e-8, 0.0)
    # each step moves p by at most lr / (1 - 0.9) in size; the 8-bit states
    # perturb the direction by a few per cent of that
    assert np.max(np.abs(p - p64)) < 0.1 * 5 * lr


def test_subnormal_scale_block_stores_zero_codes():
    rng = np.random.default_rng(3)
    n = 512
    g = rng.standard_normal(n).astype(np.float32)
    g[256:] *= np.float32(1e-20)  # v = (1 - b2) g^2 ~ 1e-43: subnormal
    z8 = np.zeros(n, np.uint8)
    zs = np.zeros(2, np.float32)
    p1, mq, vq, sm, sv = oa.step(np.zeros(n, np.float32), g, z8, z8, zs, zs, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert 0 < sv[1] < 2.0 ** -126 and sv[0] > 2.0 ** -126
    assert np.all(vq[256:] == 0) and np.count_nonzero(vq[:256]) > 200
    # m = 0.1 g ~ 1e-21 is normal: its block keeps non-zero codes
    assert sm[1] > 2.0 ** -126 and np.count_nonzero(mq[256:]) > 200
