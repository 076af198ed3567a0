"""RMS normalisation before a quantised linear layer (oracle; test use only).

Follows page 2 ("Show HN: LoRA over GGUF ..."), section "Things involved in
the training", which lists Liger Kernel's RMSNorm among the kernels of the
training path.  The pages give no formula; this is the usual definition of
RMS normalisation with a per-feature weight, in float64:

    r_t = 1 / sqrt(mean_i x[t, i]^2 + eps)
    y[t, i] = x[t, i] * r_t * w[i]

The weight w belongs to the frozen base model, so the backward returns the
input gradient only:

    dx[t, j] = r_t w_j dy[t, j] - (r_t^3 / H) x[t, j] sum_i dy[t, i] w_i x[t, i]
"""
from __future__ import annotations

import numpy as np


def forward(x: np.ndarray, w: np.ndarray, eps: float):
    """x [T, H], w [H].  Returns (y [T, H], rstd [T])."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=1) + float(eps))
    y = x * rstd[:, None] * w[None, :]
    return y, rstd


def backward(x: np.ndarray, w: np.ndarray, dy: np.ndarray, eps: float) -> np.ndarray:
    """dL/dx for the upstream gradient dy [T, H] (rstd recomputed from x)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    dy = np.asarray(dy, np.float64)
    H = x.shape[1]
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=1) + float(eps))
    inner = np.sum(dy * w[None, :] * x, axis=1)
    return rstd[:, None] * w[None, :] * dy - (rstd ** 3 / H)[:, None] * x * inner[:, None]
