"""Routed MoE FFN over block-quantised experts with per-expert LoRA adapters
(oracle; test use only).

Follows page 2 ("Show HN: LoRA over GGUF ..."), section "Things involved in
the training": quantised products over the GGUF experts grouped by expert,
after llama.cpp's grouped MMQ; per-expert adapters, which the pages run with
AITER's grouped GEMMs since they are not quantised; top-k routing after
triton-kernels; Unsloth's fast LoRA backward, which the pages apply to MoE
layers as well as linear ones; and no load-balancing loss.  The ai-manual.ru page describes
the fused MoE kernel as touching only active experts and combining the
experts' outputs with a sparse reduce.

Expert e (SwiGLU, no shared expert, one scale s for all three projections):
    g = X deq(Wg)^T + s (X Ag^T) Bg^T,   u likewise with (Wu, Au, Bu)
    h = silu(g) * u
    o = h deq(Wd)^T + s (h Ad^T) Bd^T
    y[t] = sum_j w[t, j] o(t, j)        (sum in slot order j = 0..k-1)

Two forward forms are given and cross-checked by the tests: `forward` runs
the experts over their rows in sorted order; `forward_bruteforce` loops over
tokens and slots.  `backward` is plain reverse-mode calculus in float64; it
returns dX, dlogits and the per-expert adapter gradients (exactly zero for
experts without rows).
"""
from __future__ import annotations

import numpy as np

from . import routing
from .blocks import act, dequant


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


class ExpertWeights:
    """Lazily decoded float64 expert weights for a `synth.make_moe` input set."""

    def __init__(self, inp: dict):
        self.inp = inp
        self._cache = {}

    def get(self, e: int):
        if e not in self._cache:
            i = self.inp
            qt, H, I = i["qtype"], i["H"], i["I"]
            self._cache[e] = (
                dequant(qt, i["wg"][e], I, H),
                dequant(qt, i["wu"][e], I, H),
                dequant(qt, i["wd"][e], H, I),
                np.asarray(i["ag"][e], np.float64), np.asarray(i["au"][e], np.float64),
                np.asarray(i["bg"][e], np.float64), np.asarray(i["bu"][e], np.float64),
                np.asarray(i["ad"][e], np.float64), np.asarray(i["bd"][e], np.float64),
            )
        return self._cache[e]

    def drop(self, e: int):
        self._cache.pop(e, None)


def expert_forward(X, ew, s):
    """One expert applied to rows X float64 [M, H]."""
    Wg, Wu, Wd, Ag, Au, Bg, Bu, Ad, Bd = ew
    xa_g = X @ Ag.T
    xa_u = X @ Au.T
    g = X @ Wg.T + s * (xa_g @ Bg.T)
    u = X @ Wu.T + s * (xa_u @ Bu.T)
    h = g * _sigmoid(g) * u
    xa_d = h @ Ad.T
    o = h @ Wd.T + s * (xa_d @ Bd.T)
    return dict(g=g, u=u, h=h, o=o, xa_g=xa_g, xa_u=xa_u, xa_d=xa_d)


def forward(inp: dict, ew: ExpertWeights | None = None, keep=True):
    """Grouped form.  Returns routing results, y [T, H] and per-row saved
    tensors (rows in sorted order) when keep=True."""
    ew = ew or ExpertWeights(inp)
    s = float(inp["scale"])
    T, H, I, E, k = inp["T"], inp["H"], inp["I"], inp["E"], inp["k"]
    ids, w, sorted_, offsets, pos = routing.route(inp["logits"], k)
    x = act(inp["x"])
    M = T * k
    rows = sorted_ // k
    o = np.zeros((M, H))
    saved = {n: np.zeros((M, I)) for n in ("g", "u", "h")} if keep else None
    xas = {n: np.zeros((M, inp["rank"])) for n in ("xa_g", "xa_u", "xa_d")} if keep else None
    for e in range(E):
        p0, p1 = offsets[e], offsets[e + 1]
        if p1 == p0:
            continue
        r = expert_forward(x[rows[p0:p1]], ew.get(e), s)
        o[p0:p1] = r["o"]
        if keep:
            for n in saved:
                saved[n][p0:p1] = r[n]
            for n in xas:
                xas[n][p0:p1] = r[n]
    wflat = w.ravel()
    y = np.zeros((T, H))
    for j in range(k):
        a = np.arange(T) * k + j
        y += wflat[a][:, None] * o[pos[a]]
    out = dict(ids=ids, w=w, sorted=sorted_, offsets=offsets, pos=pos, y=y, o=o)
    if keep:
        out.update(saved)
        out.update(xas)
    return out


def forward_bruteforce(inp: dict, ew: ExpertWeights | None = None, tokens=None):
    """Per-token loop: y[t] = sum_j w[t,j] * FFN_{ids[t,j]}(x[t])."""
    ew = ew or ExpertWeights(inp)
    s = float(inp["scale"])
    k = inp["k"]
    ids, w = routing.topk(inp["logits"], k)
    x = act(inp["x"])
    tokens = range(inp["T"]) if tokens is None else tokens
    y = {}
    for t in tokens:
        acc = np.zeros(inp["H"])
        for j in range(k):
            r = expert_forward(x[t:t + 1], ew.get(int(ids[t, j])), s)
            acc += w[t, j] * r["o"][0]
        y[int(t)] = acc
    return ids, w, y


def backward(inp: dict, fwd: dict, ew: ExpertWeights | None = None):
    """Reverse mode of `forward` for upstream gradient dY = inp['dy'] (bf16).

    Returns dx [T, H], dlogits [T, E], dw [T, k], the SwiGLU input gradients
    dg, du [T*k, I] (rows in sorted order) and adapter gradients
    dAg, dAu [E, r, H]; dBg, dBu [E, I, r]; dAd [E, r, I]; dBd [E, H, r]."""
    ew = ew or ExpertWeights(inp)
    s = float(inp["scale"])
    T, H, I, E, k, r = inp["T"], inp["H"], inp["I"], inp["E"], inp["k"], inp["rank"]
    dy = act(inp["dy"])
    x = act(inp["x"])
    sorted_, offsets, pos, w = fwd["sorted"], fwd["offsets"], fwd["pos"], fwd["w"]
    wflat = w.ravel()
    M = T * k
    dxrows = np.zeros((M, H))
    dw_flat = np.zeros(M)
    dg_rows = np.zeros((M, I))
    du_rows = np.zeros((M, I))
    g = dict(dAg=np.zeros((E, r, H)), dAu=np.zeros((E, r, H)), dBg=np.zeros((E, I, r)),
             dBu=np.zeros((E, I, r)), dAd=np.zeros((E, r, I)), dBd=np.zeros((E, H, r)))
    for e in range(E):
        p0, p1 = offsets[e], offsets[e + 1]
        if p1 == p0:
            continue
        Wg, Wu, Wd, Ag, Au, Bg, Bu, Ad, Bd = ew.get(e)
        a = sorted_[p0:p1]
        t = a // k
        X = x[t]
        dY = dy[t]
        wv = wflat[a][:, None]
        # gate weight gradient: <dY[t], o>
        dw_flat[a] = (dY * fwd["o"][p0:p1]).sum(axis=1)
        dO = wv * dY
        hh, gg, uu = fwd["h"][p0:p1], fwd["g"][p0:p1], fwd["u"][p0:p1]
        dOB = dO @ Bd
        dh = dO @ Wd + s * (dOB @ Ad)
        g["dBd"][e] = s * (dO.T @ fwd["xa_d"][p0:p1])
        g["dAd"][e] = s * (dOB.T @ hh)
        sg = _sigmoid(gg)
        dg = dh * uu * sg * (1.0 + gg * (1.0 - sg))
        du = dh * gg * sg
        dg_rows[p0:p1] = dg
        du_rows[p0:p1] = du
        dgB = dg @ Bg
        duB = du @ Bu
        dxrows[p0:p1] = dg @ Wg + du @ Wu + s * (dgB @ Ag + duB @ Au)
        g["dBg"][e] = s * (dg.T @ fwd["xa_g"][p0:p1])
        g["dBu"][e] = s * (du.T @ fwd["xa_u"][p0:p1])
        g["dAg"][e] = s * (dgB.T @ X)
        g["dAu"][e] = s * (duB.T @ X)
    dx = np.zeros((T, H))
    for j in range(k):
        a = np.arange(T) * k + j
        dx += dxrows[pos[a]]
    dw = dw_flat.reshape(T, k)
    dlogits = routing.backward(fwd["ids"], w, dw, E)
    out = dict(dx=dx, dlogits=dlogits, dw=dw, dg=dg_rows, du=du_rows)
    out.update(g)
    return out


def expert_backward_rows(inp: dict, e: int, rows_a: np.ndarray, w_rows: np.ndarray,
                         ew: ExpertWeights):
    """Adapter gradients of one expert from its assignments `rows_a` (flat
    indices t*k+j, in sorted order) with gate weights `w_rows`.  Used by the
    sampled full-size checks, which need one expert at a time."""
    s = float(inp["scale"])
    k = inp["k"]
    x = act(inp["x"])
    dy = act(inp["dy"])
    Wg, Wu, Wd, Ag, Au, Bg, Bu, Ad, Bd = ew.get(e)
    t = np.asarray(rows_a) // k
    X = x[t]
    f = expert_forward(X, ew.get(e), s)
    dO = np.asarray(w_rows, np.float64)[:, None] * dy[t]
    dOB = dO @ Bd
    dh = dO @ Wd + s * (dOB @ Ad)
    sg = _sigmoid(f["g"])
    dg = dh * f["u"] * sg * (1.0 + f["g"] * (1.0 - sg))
    du = dh * f["g"] * sg
    dgB = dg @ Bg
    duB = du @ Bu
    return dict(dBd=s * (dO.T @ f["xa_d"]), dAd=s * (dOB.T @ f["h"]),
                dBg=s * (dg.T @ f["xa_g"]), dBu=s * (du.T @ f["xa_u"]),
                dAg=s * (dgB.T @ X), dAu=s * (duB.T @ X),
                dxrows=dg @ Wg + du @ Wu + s * (dgB @ Ag + duB @ Au),
                dw=(dy[t] * f["o"]).sum(axis=1), y_rows=f["o"], dg=dg, du=du,
                g=f["g"], u=f["u"], h=f["h"])
