"""Float32 model of the 8-bit AdamW kernel's arithmetic (a kernel
regression check, NOT the oracle).

The oracle (oracle/adamw8bit.py) defines the step in float64 and the GPU
parity test checks the kernel against it within float32 error bounds.  This
module instead repeats the kernel's own float32 operations in its order
(one division per element with host constants k2 = 1/sqrt(1 - b2^t),
kd = 1 - lr wd, s1 = lr/(1 - b1^t); states normalised by the float32
reciprocal of the block scale; no fused multiply-adds), so that a change of
the kernel's arithmetic shows up as a bit difference.  It is test
infrastructure like the oracle and shares no code with the library.
"""
from __future__ import annotations

import numpy as np

BLOCK = 256
F32 = np.float32


# 10^-e as double literals (each the double nearest to the decimal value)
_DECADE = (1.0, 0.1, 0.01, 0.001, 0.0001, 0.00001, 0.000001, 0.0000001)


def _magnitudes(bits: int) -> np.ndarray:
    """Values of the magnitude codes 0 .. 2^bits - 1: the rule evaluated in
    double precision in the order written, then rounded to float32."""
    out = np.zeros(1 << bits, np.float64)
    for code in range(1, 1 << bits):
        top = code.bit_length() - 1      # position of the indicator bit
        e = bits - 1 - top                # leading zeros
        f = top                           # fraction bits below the indicator
        i = code - (1 << top)
        out[code] = _DECADE[e] * (0.1 + 0.9 * ((i + 1) / (1 << f)))
    return out


def signed_table() -> np.ndarray:
    """float32 [256]: code c = sign bit 7 | magnitude bits 0..6."""
    mag = _magnitudes(7)
    t = np.concatenate([mag, -mag])
    return t.astype(F32)


def unsigned_table() -> np.ndarray:
    return _magnitudes(8).astype(F32)


def quantize(xn: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Nearest code of each float32 value in xn (ties: smaller magnitude)."""
    xn = np.asarray(xn, F32)
    order = np.argsort(table, kind="stable")
    vals = table[order]
    # drop the duplicate -0 of the signed table: keep the first of equal values
    keep = np.concatenate([[True], vals[1:] != vals[:-1]])
    vals, order = vals[keep], order[keep]
    hi = np.searchsorted(vals, xn, side="left")
    hi = np.clip(hi, 0, vals.size - 1)
    lo = np.clip(hi - 1, 0, vals.size - 1)
    dlo = np.abs(xn - vals[lo]).astype(F32)
    dhi = np.abs(vals[hi] - xn).astype(F32)
    pick_hi = dhi < dlo
    tie = dhi == dlo
    # on a tie take the code of smaller magnitude
    pick_hi = pick_hi | (tie & (np.abs(vals[hi]) < np.abs(vals[lo])))
    idx = np.where(pick_hi, hi, lo)
    return order[idx].astype(np.uint8)


def dequantize(codes: np.ndarray, scale: np.ndarray, table: np.ndarray, n: int) -> np.ndarray:
    """float32 [n] from codes [n] and block scales [ceil(n / 256)]."""
    s = np.repeat(np.asarray(scale, F32), BLOCK)[:n]
    return (table[np.asarray(codes, np.int64)] * s).astype(F32)


def step(p, g, mq, vq, sm, sv, t: int, lr: float, b1: float, b2: float, eps: float, wd: float):
    """One AdamW step on float32 p [n] with gradient g [n] and 8-bit states
    (mq, vq uint8 [n]; sm, sv float32 [nblk]).  Returns new (p, mq, vq, sm, sv)."""
    # hyper-parameters are float32 values (the kernel's argument type); the
    # derived constants come from them in double precision, rounded once
    lr, b1, b2, eps, wd = (float(F32(x)) for x in (lr, b1, b2, eps, wd))
    ts, tu = signed_table(), unsigned_table()
    p = np.asarray(p, F32).copy()
    g = np.asarray(g, F32)
    n = p.size
    m = dequantize(mq, sm, ts, n)
    v = dequantize(vq, sv, tu, n)
    b1f, b2f = F32(b1), F32(b2)
    om1, om2 = F32(1.0 - b1), F32(1.0 - b2)
    k2 = F32(1.0 / np.sqrt(1.0 - b2 ** t))
    kd = F32(1.0 - lr * wd)
    s1 = F32(lr / (1.0 - b1 ** t))
    epsf = F32(eps)
    m = (b1f * m + om1 * g).astype(F32)
    v = (b2f * v + om2 * (g * g)).astype(F32)
    d = (np.sqrt(v) * k2 + epsf).astype(F32)
    p = (p * kd - s1 * (m / d).astype(F32)).astype(F32)
    nblk = (n + BLOCK - 1) // BLOCK
    pad = nblk * BLOCK - n
    am = np.pad(np.abs(m), (0, pad)).reshape(nblk, BLOCK).max(axis=1).astype(F32)
    av = np.pad(v, (0, pad)).reshape(nblk, BLOCK).max(axis=1).astype(F32)
    # per-block reciprocal scales; below the smallest normal float32 the
    # block normalises to 0
    tiny = F32(2.0 ** -126)
    rm = np.where(am >= tiny, F32(1) / np.where(am >= tiny, am, F32(1)), F32(0)).astype(F32)
    rv = np.where(av >= tiny, F32(1) / np.where(av >= tiny, av, F32(1)), F32(0)).astype(F32)
    mn = (m * np.repeat(rm, BLOCK)[:n]).astype(F32)
    vn = (v * np.repeat(rv, BLOCK)[:n]).astype(F32)
    return p, quantize(mn, ts), quantize(vn, tu), am, av
