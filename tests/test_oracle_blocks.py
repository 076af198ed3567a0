"""Pins for the oracle's block decode (CPU only).

* hand-built blocks with values worked out from the definitions
  (tests/golden/dequant_handbuilt.txt)
* quantise -> decode round trip within the error the quantiser's rule allows
  (the quantiser lives in synth/ and is written independently of the decode)
* row/block layout: a matrix whose blocks each carry their own index
"""
import numpy as np
import pytest

import synth
from oracle import blocks as ob


def _same(got, exp):
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    nan_g, nan_e = np.isnan(got), np.isnan(exp)
    assert (nan_g == nan_e).all(), (got, exp)
    ok = ~nan_e
    assert (got[ok] == exp[ok]).all(), (got, exp)  # +0 == -0 as intended


def test_golden_cases(golden_blocks):
    assert len(golden_blocks) >= 10
    for c in golden_blocks:
        bs = ob.BLOCK_BYTES[c["qtype"]]
        assert len(c["bytes"]) == bs, c["name"]
        raw = np.frombuffer(c["bytes"], np.uint8)
        got = ob.dequant_f32(c["qtype"], raw, 1, 32)[0]
        _same(got, c["expect"])


def test_golden_exact_value_rounds_once():
    # the q2 single-rounding case: exact value is 1 + 3*2^-24, float32 result 1 + 2^-22
    raw = np.frombuffer(bytes.fromhex("003c0300e4e4e4e4e4e4e4e4"), np.uint8)
    exact = ob.dequant(2, raw, 1, 32)[0]
    assert exact[8] == 1.0 + 3.0 * 2.0 ** -24
    assert np.float32(exact[8]) == np.float32(1.0 + 2.0 ** -22)


@pytest.mark.parametrize("qtype", [0, 1, 2])
def test_roundtrip_bound(qtype):
    rng = np.random.default_rng(7)
    w = (0.02 * rng.standard_normal((64, 256))).astype(np.float32)
    w[3, :32] = 0.0  # an all-zero block
    w[5, 32:64] = 1e-3  # a constant block
    raw = synth.quantize(qtype, w)
    got = ob.dequant(qtype, raw, 64, 256)
    b = w.reshape(64, 8, 32).astype(np.float64)
    err = np.abs(got.reshape(64, 8, 32) - b)
    if qtype == 0:
        d32 = np.abs(b).max(axis=2) / 127.0
        d16 = d32.astype(np.float16).astype(np.float64)
        bound = d32 / 2 + 127 * np.abs(d16 - d32) + 1e-12
    elif qtype == 1:
        idx = np.abs(b).argmax(axis=2)
        mx = np.take_along_axis(b, idx[..., None], axis=2)[..., 0]
        d32 = np.abs(mx) / 8.0
        d16 = d32.astype(np.float16).astype(np.float64)
        # largest |w| maps to q in {0, 15}: at most one step of d plus the scale rounding
        bound = d32 + 8 * np.abs(d16 - d32) + 1e-12
    else:
        lo, hi = b.min(axis=2), b.max(axis=2)
        d32 = (hi - lo) / 3.0
        d16 = d32.astype(np.float16).astype(np.float64)
        m16 = lo.astype(np.float16).astype(np.float64)
        bound = d32 / 2 + 3 * np.abs(d16 - d32) + np.abs(m16 - lo) + 1e-12
    assert (err <= bound[..., None]).all()
    # zero block decodes to exactly zero
    assert np.all(got[3, :32] == 0.0)


@pytest.mark.parametrize("qtype", [0, 1, 2])
def test_row_block_layout(qtype):
    """Every block of a 3 x 96 matrix holds its own exactly-representable
    pattern (unit 2^-j for block j, distinct integer codes), built so the
    quantiser reproduces it exactly; any mix-up of rows, blocks or element
    order changes the decoded matrix."""
    rows, nb = 3, 3
    w = np.zeros((rows, nb * 32), np.float64)
    for r in range(rows):
        for b in range(nb):
            j = r * nb + b
            u = 2.0 ** -(j % 8)
            i = np.arange(32)
            if qtype == 0:
                q = (i * 5 + j) % 127 - 63
                q[0] = 127
                v = q * u
            elif qtype == 1:
                q = 1 + (i * 3 + j) % 15
                q[0] = 0
                v = (q - 8) * u
            else:
                q = (i + j) % 4
                q[0], q[1] = 0, 3
                v = -0.25 * j + q * u
            w[r, b * 32:(b + 1) * 32] = v
    raw = synth.quantize(qtype, w.astype(np.float32))
    got = ob.dequant(qtype, raw, rows, nb * 32)
    assert np.array_equal(got, w)


def test_ramp_element_order():
    """Q8_0 ramp over 4 blocks: w = q*d with d = 1 for every block."""
    raw = np.zeros((1, 4, 34), np.uint8)
    raw[..., 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    q = (np.arange(128) - 64).astype(np.int8).reshape(4, 32)
    raw[0, :, 2:] = q.view(np.uint8)
    got = ob.dequant(0, raw.reshape(1, -1), 1, 128)[0]
    assert np.array_equal(got, np.arange(128) - 64.0)


def test_bf16_value_exact():
    bits = synth.f32_to_bf16_bits(np.array([1.0, -2.5, 3.1415927, 1e-40, 65504.0], np.float32))
    v = ob.bf16_value(bits)
    assert v[0] == 1.0 and v[1] == -2.5
    assert v[2] == 3.140625  # 3.1415927 rounded to 8 significant bits
    assert v[4] == 65536.0
