"""Block decode, written from the block definitions (oracle; test use only).

The pages train over a GGUF base read by quantised matrix products after
llama.cpp's MMQ (page 2, "Things involved in the training"), i.e. the weights stay as blocks of 32
small integers with fp16 scale(s).  Three formats are decoded:

* Q8_0  (34 bytes): fp16 d, then 32 signed bytes q;            w_i = d*q_i
* Q4_0  (18 bytes): fp16 d, then 16 bytes; byte j carries element j in its
  low nibble and element j+16 in its high nibble;               w_i = d*(q_i-8)
* Q2_DM (12 bytes): fp16 d, fp16 m, then 8 bytes; byte j carries element
  j+8p in bits [2p, 2p+2) for p = 0..3;                         w_i = d*q_i + m

(The 2-bit scale/min format stands in for the pages' 2-bit bases, page 2,
sections "DeepSeek-specific" and "Qwen4-Exp-specific".)  All multi-byte fields
are little-endian, blocks of one row are contiguous, rows are contiguous.

`dequant` returns the exact real value of every weight as float64 (every
product and the one sum are exact in float64 for fp16 operands);
`dequant_f32` rounds that value once to float32 (round to nearest even), which
is the unique correctly-rounded float32 result.
"""
from __future__ import annotations

import numpy as np

Q8_0, Q4_0, Q2_DM = 0, 1, 2
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q2_DM: 12}


def _fp16_le(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    bits = lo.astype(np.uint16) | (hi.astype(np.uint16) << np.uint16(8))
    return bits.view(np.float16).astype(np.float64)


def dequant(qtype: int, blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Exact decode of `rows` x `cols` weights from raw block bytes -> float64."""
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    bs = BLOCK_BYTES[qtype]
    nb = cols // 32
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(rows, nb, bs)
    d = _fp16_le(b[..., 0], b[..., 1])
    if qtype == Q8_0:
        q = b[..., 2:34].view(np.int8).astype(np.float64)
        w = d[..., None] * q
    elif qtype == Q4_0:
        qs = b[..., 2:18]
        q = np.concatenate([qs & 0x0F, qs >> 4], axis=-1).astype(np.float64)
        w = d[..., None] * (q - 8.0)
    elif qtype == Q2_DM:
        m = _fp16_le(b[..., 2], b[..., 3])
        qs = b[..., 4:12]
        q = np.concatenate([(qs >> (2 * p)) & 0x3 for p in range(4)], axis=-1).astype(np.float64)
        w = d[..., None] * q + m[..., None]
    else:
        raise ValueError(f"unknown qtype {qtype}")
    return w.reshape(rows, cols)


def dequant_f32(qtype: int, blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Decode rounded once to float32 (RNE)."""
    with np.errstate(over="ignore", invalid="ignore"):
        return dequant(qtype, blocks, rows, cols).astype(np.float32)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def act(v: np.ndarray) -> np.ndarray:
    """Activations arrive as bf16 bit patterns (uint16); float arrays (used by
    the finite-difference pins) pass through as float64."""
    v = np.asarray(v)
    if v.dtype == np.uint16:
        return bf16_value(v)
    return v.astype(np.float64)
