"""AdamW with 8-bit block-wise quantised states (oracle; test use only).

Follows page 2 ("Show HN: LoRA over GGUF ..."), section "Things involved in
the training", which names bitsandbytes' 8-bit AdamW as the optimizer of the
adapters.  The pages give no formulas; the reading used here is the
textbook AdamW step with decoupled weight decay, taken on states that are
stored as 8-bit codes with one scale per block, everything in float64:

* State storage.  256 consecutive elements form a block.  A block stores
  one float32 scale per state (the block's largest |m|, or largest v) and
  one 8-bit code per element; the element's state is book[code] * scale.
* Code books ("dynamic tree" layout): an optional sign bit, then e zero
  bits, a one bit and f fraction bits i; the value is
  10^-e * (0.1 + 0.9 * (i + 1) / 2^f), and the all-zero magnitude is 0.
  Signed book (for m): sign bit 7 + 7 magnitude bits, e = 0..6, f = 6 - e.
  Unsigned book (for v): 8 magnitude bits, e = 0..7, f = 7 - e.
  The books here are the real numbers of that rule (float64).
* One step t >= 1 with gradient g, on the dequantised states m, v:
      m' = b1 m + (1 - b1) g,   v' = b2 v + (1 - b2) g^2
      p' = p - lr * ( m'/(1 - b1^t) / (sqrt(v'/(1 - b2^t)) + eps) + wd p )
  The hyper-parameters are the float32 values the caller passes.
* New storage: scale_m = max |m'| and scale_v = max v' over the block,
  stored as float32 (round to nearest); each code is the book entry
  nearest to m' / scale_m (v' / scale_v), ties to the smaller magnitude.
  A block whose scale is below the smallest normal float32 (2^-126, zero
  included) stores code 0 for every element (such states are far below any
  eps and do not move p).  p' is stored as float32 (round to nearest).

The GPU kernel takes these steps in float32; its results are compared with
the float64 values here within float32 error bounds (see the tests).
"""
from __future__ import annotations

import numpy as np

BLOCK = 256
TINY = 2.0 ** -126


def _magnitudes(bits: int) -> np.ndarray:
    """Values of the magnitude codes 0 .. 2^bits - 1 of a book (float64)."""
    out = np.zeros(1 << bits, np.float64)
    for code in range(1, 1 << bits):
        top = code.bit_length() - 1      # position of the indicator bit
        e = bits - 1 - top                # zero bits above it
        f = top                           # fraction bits below it
        i = code - (1 << top)
        out[code] = 10.0 ** (-e) * (0.1 + 0.9 * (i + 1) / 2.0 ** f)
    return out


def signed_table() -> np.ndarray:
    """float64 [256]: code c = sign bit 7 | magnitude bits 0..6."""
    mag = _magnitudes(7)
    return np.concatenate([mag, -mag])


def unsigned_table() -> np.ndarray:
    return _magnitudes(8)


def _sorted_book(table: np.ndarray):
    order = np.argsort(table, kind="stable")
    vals = table[order]
    # the signed book holds 0 twice (+0 and -0): keep the first (code 0)
    keep = np.concatenate([[True], vals[1:] != vals[:-1]])
    return vals[keep], order[keep]


def quantize(xn: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Nearest code of each value in xn (ties: smaller magnitude)."""
    xn = np.asarray(xn, np.float64)
    vals, order = _sorted_book(table)
    hi = np.clip(np.searchsorted(vals, xn, side="left"), 0, vals.size - 1)
    lo = np.clip(hi - 1, 0, vals.size - 1)
    dlo = np.abs(xn - vals[lo])
    dhi = np.abs(vals[hi] - xn)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (np.abs(vals[hi]) < np.abs(vals[lo])))
    return order[np.where(pick_hi, hi, lo)].astype(np.uint8)


def neighbours(xn: np.ndarray, table: np.ndarray):
    """For each value: the codes of the book entries just below and just
    above it (equal when the value is a book entry or outside the book), and
    the distance of the value from the midpoint between those two entries."""
    xn = np.asarray(xn, np.float64)
    vals, order = _sorted_book(table)
    hi = np.clip(np.searchsorted(vals, xn, side="left"), 0, vals.size - 1)
    lo = np.where(vals[hi] > xn, np.clip(hi - 1, 0, vals.size - 1), hi)
    mid = 0.5 * (vals[lo] + vals[hi])
    return order[lo].astype(np.uint8), order[hi].astype(np.uint8), np.abs(xn - mid)


def dequantize(codes: np.ndarray, scale: np.ndarray, table: np.ndarray, n: int) -> np.ndarray:
    """float64 [n] states from codes [n] and block scales [ceil(n / 256)]."""
    s = np.repeat(np.asarray(scale, np.float64), BLOCK)[:n]
    return table[np.asarray(codes, np.int64)] * s


def _block_max(a: np.ndarray) -> np.ndarray:
    n = a.size
    nblk = (n + BLOCK - 1) // BLOCK
    return np.pad(a, (0, nblk * BLOCK - n)).reshape(nblk, BLOCK).max(axis=1)


def step_exact(p, g, mq, vq, sm, sv, t: int, lr: float, b1: float, b2: float, eps: float, wd: float):
    """One step in float64 from the stored state (p float32 [n], g float32
    [n], codes uint8 [n], scales float32 [nblk]).  Returns a dict of float64
    results before storage rounding: p, m, v (new states), scale_m, scale_v
    (block maxima), mn, vn (states divided by their block's scale, 0 where
    the scale is below 2^-126) and m_in, v_in (the dequantised old states)."""
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (lr, b1, b2, eps, wd))
    p = np.asarray(p, np.float32).astype(np.float64)
    g = np.asarray(g, np.float32).astype(np.float64)
    n = p.size
    m_in = dequantize(mq, sm, signed_table(), n)
    v_in = dequantize(vq, sv, unsigned_table(), n)
    m = b1 * m_in + (1.0 - b1) * g
    v = b2 * v_in + (1.0 - b2) * g * g
    mhat = m / (1.0 - b1 ** t)
    vhat = v / (1.0 - b2 ** t)
    p_new = p - lr * (mhat / (np.sqrt(vhat) + eps) + wd * p)
    scale_m = _block_max(np.abs(m))
    scale_v = _block_max(v)
    rs_m = np.repeat(scale_m, BLOCK)[:n]
    rs_v = np.repeat(scale_v, BLOCK)[:n]
    mn = np.where(rs_m >= TINY, m / np.where(rs_m >= TINY, rs_m, 1.0), 0.0)
    vn = np.where(rs_v >= TINY, v / np.where(rs_v >= TINY, rs_v, 1.0), 0.0)
    return {"p": p_new, "p_in": p, "m": m, "v": v, "scale_m": scale_m, "scale_v": scale_v, "mn": mn, "vn": vn,
            "m_in": m_in, "v_in": v_in, "g": g, "b1": b1, "b2": b2, "lr": lr, "eps": eps, "wd": wd, "t": t}


def step(p, g, mq, vq, sm, sv, t: int, lr: float, b1: float, b2: float, eps: float, wd: float):
    """One step with the results stored: (p float32, m codes, v codes,
    m scales float32, v scales float32)."""
    r = step_exact(p, g, mq, vq, sm, sv, t, lr, b1, b2, eps, wd)
    return (r["p"].astype(np.float32), quantize(r["mn"], signed_table()),
            quantize(r["vn"], unsigned_table()), r["scale_m"].astype(np.float32),
            r["scale_v"].astype(np.float32))
