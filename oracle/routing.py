"""MoE routing (oracle; test use only).

Follows page 2 ("Show HN: LoRA over GGUF ..."), section "Things involved in
the training", which names OpenAI's triton-kernels as the model for the
MoE routing and turns the load-balancing loss off (same section), so the
router gradient is that of the gate weights alone.

Per token t over the E router logits l:
  1. the k experts with the largest logits, ties broken toward the lower
     expert index, listed in that order -> ids[t, 0..k-1];
  2. gate weights = softmax over the k selected logits (equal to a softmax
     over all E followed by top-k and renormalisation);
  3. assignments a = t*k + j are sorted stably by expert -> sorted;
  4. offsets[e] = number of assignments with expert < e  (E + 1 entries);
  5. pos[sorted[p]] = p.
Backward: with dw the gradient of the gate weights,
  dlogits[t, ids[t, j]] = w[t, j] * (dw[t, j] - sum_i w[t, i] dw[t, i]),
and zero at every unselected expert.
"""
from __future__ import annotations

import numpy as np


def topk(logits: np.ndarray, k: int):
    # fp32 router logits widen exactly to float64; float64 inputs (finite-
    # difference pins) are used as they are
    logits = np.asarray(logits).astype(np.float64)
    T, E = logits.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -logits), axis=-1)
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


def sort_assignments(ids: np.ndarray, E: int):
    flat = np.asarray(ids, np.int64).ravel()
    sorted_ = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    pos = np.empty(flat.size, np.int32)
    pos[sorted_] = np.arange(flat.size, dtype=np.int32)
    return sorted_, offsets, pos


def route(logits: np.ndarray, k: int):
    """Returns ids int32 [T,k], w float64 [T,k], sorted int32 [T*k],
    offsets int32 [E+1], pos int32 [T*k]."""
    E = np.asarray(logits).shape[1]
    ids, w = topk(logits, k)
    sorted_, offsets, pos = sort_assignments(ids, E)
    return ids, w, sorted_, offsets, pos


def backward(ids: np.ndarray, w: np.ndarray, dw: np.ndarray, E: int) -> np.ndarray:
    T, k = ids.shape
    w = np.asarray(w, np.float64)
    dw = np.asarray(dw, np.float64)
    inner = (w * dw).sum(axis=1, keepdims=True)
    g = w * (dw - inner)
    dl = np.zeros((T, E), np.float64)
    np.put_along_axis(dl, np.asarray(ids, np.int64), g, axis=1)
    return dl
