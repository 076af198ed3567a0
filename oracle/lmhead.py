"""LM head over a block-quantised W_out with a LoRA adapter and chunked
cross entropy (oracle; test use only).

Follows page 2 ("Show HN: LoRA over GGUF ..."), section "Things involved in
the training", which lists a chunked cross entropy after Liger Kernel's,
computed over the MMQ output: the [tokens x vocab] logits are never held
whole; the vocabulary is walked in row chunks with an online log-sum-exp.

    z      = h deq(W)^T + s (h A^T) B^T                 (per chunk of rows)
    m, l   : m' = max(m, max_v z),  l' = l e^(m - m') + sum_v e^(z - m')
    lse    = m + ln l
    loss   = (1/N_valid) sum_{t valid} (lse_t - z[t, label_t])
    G      = (g_out / N_valid) (softmax(z) - onehot(label)), rows of ignored
             tokens are zero
    dh     = G deq(W) + s (G B) A,   dB = s G^T (h A^T),   dA = s (G B)^T h

Ignored tokens carry label == ignore_index.  With no valid token the loss and
all gradients are defined as zero.  `forward_backward_direct` forms the full
logits at once and is the cross-check for the chunked walk.
"""
from __future__ import annotations

import numpy as np

from .blocks import act, dequant


def _chunks(V: int, chunk: int):
    c0 = 0
    while c0 < V:
        yield c0, min(V, c0 + chunk)
        c0 += chunk


def forward_backward(inp: dict, chunk: int | None = None, ignore_index: int = -100,
                     g_out: float = 1.0, want_grad: bool = True, W_full=None):
    h = act(inp["h"])
    T, H, V = inp["T"], inp["H"], inp["V"]
    A = np.asarray(inp["A"], np.float64)
    B = np.asarray(inp["B"], np.float64)
    s = float(inp["scale"])
    labels = np.asarray(inp["labels"], np.int64)
    chunk = chunk or inp.get("chunk", 4096)
    bs = inp["blocks"]

    def Wc(c0, c1):
        if W_full is not None:
            return W_full[c0:c1]
        return dequant(inp["qtype"], bs[c0:c1], c1 - c0, H)

    valid = labels != ignore_index
    nv = int(valid.sum())
    xa = h @ A.T
    m = np.full(T, -np.inf)
    l = np.zeros(T)
    zlab = np.zeros(T)
    for c0, c1 in _chunks(V, chunk):
        z = h @ Wc(c0, c1).T + s * (xa @ B[c0:c1].T)
        mn = np.maximum(m, z.max(axis=1))
        l = l * np.exp(m - mn) + np.exp(z - mn[:, None]).sum(axis=1)
        m = mn
        inside = valid & (labels >= c0) & (labels < c1)
        ti = np.nonzero(inside)[0]
        zlab[ti] = z[ti, labels[ti] - c0]
    lse = m + np.log(l)
    loss = float((lse - zlab)[valid].sum() / nv) if nv else 0.0
    out = dict(loss=loss, lse=lse, n_valid=nv, xa=xa)
    if not want_grad:
        return out
    dh = np.zeros((T, H))
    dB = np.zeros((V, A.shape[0]))
    GB = np.zeros((T, A.shape[0]))
    coef = (g_out / nv) if nv else 0.0
    for c0, c1 in _chunks(V, chunk):
        W = Wc(c0, c1)
        z = h @ W.T + s * (xa @ B[c0:c1].T)
        G = np.exp(z - lse[:, None])
        inside = valid & (labels >= c0) & (labels < c1)
        ti = np.nonzero(inside)[0]
        G[ti, labels[ti] - c0] -= 1.0
        G *= coef
        G[~valid] = 0.0
        dh += G @ W
        dB[c0:c1] = s * (G.T @ xa)
        GB += G @ B[c0:c1]
    dh += s * (GB @ A)
    dA = s * (GB.T @ h)
    out.update(dh=dh, dA=dA, dB=dB)
    return out


def forward_backward_direct(inp: dict, ignore_index: int = -100, g_out: float = 1.0):
    """Unchunked reference: full logits, direct log-sum-exp."""
    h = act(inp["h"])
    T, H, V = inp["T"], inp["H"], inp["V"]
    A = np.asarray(inp["A"], np.float64)
    B = np.asarray(inp["B"], np.float64)
    s = float(inp["scale"])
    labels = np.asarray(inp["labels"], np.int64)
    W = dequant(inp["qtype"], inp["blocks"], V, H)
    z = h @ W.T + s * (h @ A.T) @ B.T
    zmax = z.max(axis=1, keepdims=True)
    lse = (zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True)))[:, 0]
    valid = labels != ignore_index
    nv = int(valid.sum())
    t = np.nonzero(valid)[0]
    loss = float((lse[t] - z[t, labels[t]]).sum() / nv) if nv else 0.0
    P = np.exp(z - lse[:, None])
    P[t, labels[t]] -= 1.0
    P[~valid] = 0.0
    G = P * ((g_out / nv) if nv else 0.0)
    dh = G @ W + s * (G @ B) @ A
    dB = s * G.T @ (h @ A.T)
    dA = s * (G @ B).T @ h
    return dict(loss=loss, lse=lse, dh=dh, dA=dA, dB=dB, n_valid=nv)
