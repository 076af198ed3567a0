"""Fused quantised linear layer with a LoRA adapter (oracle; test use only).

Follows page 2 ("Show HN: LoRA over GGUF ..."), section "Things involved in
the training": the base product is a quantised matrix product over the
frozen block-quantised W, after llama.cpp's MMQ, and the backward is
Unsloth's fast LoRA formula for a linear layer: the gradient never forms
B.A and the frozen W receives no gradient.

With s the adapter scale (alpha / rank), A [r, K], B [N, r]:
    xa = x A^T
    y  = x deq(W)^T + s xa B^T
    dX = dY deq(W) + s (dY B) A
    dB = s dY^T xa
    dA = s (dY B)^T x
All arithmetic is float64 on the exact input values.
"""
from __future__ import annotations

import numpy as np

from .blocks import act, dequant


def weights(qtype: int, blocks: np.ndarray, n_out: int, n_in: int) -> np.ndarray:
    return dequant(qtype, blocks, n_out, n_in)


def forward(x: np.ndarray, W: np.ndarray, A: np.ndarray, B: np.ndarray, s: float):
    """x float64 [T, K]; W float64 [N, K].  Returns (y [T, N], xa [T, r])."""
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    xa = x @ A.T
    y = x @ W.T + float(s) * (xa @ B.T)
    return y, xa


def backward(x: np.ndarray, dy: np.ndarray, W: np.ndarray, A: np.ndarray, B: np.ndarray,
             s: float):
    """Returns (dX [T, K], dA [r, K], dB [N, r]).  xa is recomputed from x."""
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    s = float(s)
    xa = x @ A.T
    dyB = dy @ B
    dx = dy @ W + s * (dyB @ A)
    dB = s * (dy.T @ xa)
    dA = s * (dyB.T @ x)
    return dx, dA, dB


def run(inp: dict):
    """Forward + backward of a `synth.make_linear` input set, in float64."""
    W = weights(inp["qtype"], inp["blocks"], inp["N"], inp["K"])
    x = act(inp["x"])
    dy = act(inp["dy"])
    y, xa = forward(x, W, inp["A"], inp["B"], inp["scale"])
    dx, dA, dB = backward(x, dy, W, inp["A"], inp["B"], inp["scale"])
    return dict(y=y, xa=xa, dx=dx, dA=dA, dB=dB)
