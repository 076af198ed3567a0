"""Pins for the oracle's routing (CPU): pure-Python brute force, hand-built
ties, degenerate k = E and E = 1, and the router backward by finite
differences of the softmax over the selected logits."""
import math

import numpy as np
import pytest

from oracle import routing as orr


def brute_route(logits, k):
    T, E = len(logits), len(logits[0])
    ids, w = [], []
    for t in range(T):
        cand = list(range(E))
        # selection sort by (value desc, index asc)
        chosen = []
        for _ in range(k):
            best = None
            for e in cand:
                if best is None or logits[t][e] > logits[t][best] or (
                        logits[t][e] == logits[t][best] and e < best):
                    best = e
            chosen.append(best)
            cand.remove(best)
        ids.append(chosen)
        m = logits[t][chosen[0]]
        ex = [math.exp(logits[t][e] - m) for e in chosen]
        z = sum(ex)
        w.append([v / z for v in ex])
    # stable bucket sort of flat assignments
    buckets = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            buckets[ids[t][j]].append(t * k + j)
    sorted_ = [a for b in buckets for a in b]
    offsets = [0]
    for b in buckets:
        offsets.append(offsets[-1] + len(b))
    pos = [0] * (T * k)
    for p, a in enumerate(sorted_):
        pos[a] = p
    return ids, w, sorted_, offsets, pos


@pytest.mark.parametrize("T,E,k,seed", [(7, 8, 2, 0), (16, 32, 8, 1), (5, 4, 4, 2), (9, 1, 1, 3),
                                        (33, 64, 8, 4)])
def test_matches_bruteforce(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w, s, off, pos = orr.route(logits, k)
    bi, bw, bs, bo, bp = brute_route(logits.astype(np.float64).tolist(), k)
    assert ids.tolist() == bi
    np.testing.assert_allclose(w, bw, rtol=1e-14)
    assert s.tolist() == bs and off.tolist() == bo and pos.tolist() == bp


def test_ties_prefer_lower_index():
    logits = np.array([[1.0, 3.0, 3.0, 0.5, 3.0],
                       [0.0, 0.0, 0.0, 0.0, 0.0],
                       [-0.0, 0.0, -1.0, -0.0, 2.0]], np.float32)
    ids, w, _, _, _ = orr.route(logits, 3)
    assert ids.tolist() == [[1, 2, 4], [0, 1, 2], [4, 0, 1]]
    np.testing.assert_allclose(w[1], [1 / 3] * 3, rtol=1e-15)
    bi = brute_route(logits.astype(np.float64).tolist(), 3)[0]
    assert ids.tolist() == bi


def test_offsets_and_pos_invariants():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((100, 16)).astype(np.float32)
    ids, w, s, off, pos = orr.route(logits, 4)
    assert off[0] == 0 and off[-1] == 400 and (np.diff(off) >= 0).all()
    assert np.array_equal(np.sort(s), np.arange(400))
    assert np.array_equal(s[pos], np.arange(400))
    flat = ids.ravel()
    for e in range(16):
        seg = s[off[e]:off[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def test_backward_finite_differences():
    rng = np.random.default_rng(6)
    T, E, k = 4, 10, 3
    logits = rng.standard_normal((T, E))
    ids, w = orr.topk(logits.astype(np.float32), k)
    logits = logits.astype(np.float32).astype(np.float64)
    dw = rng.standard_normal((T, k))
    dl = orr.backward(ids, w, dw, E)

    def L(lg):
        sel = np.take_along_axis(lg, ids.astype(np.int64), axis=1)
        ex = np.exp(sel - sel.max(axis=1, keepdims=True))
        return float((dw * ex / ex.sum(axis=1, keepdims=True)).sum())

    h = 1e-5
    for t in range(T):
        for e in range(E):
            p = logits.copy(); p[t, e] += h
            m = logits.copy(); m[t, e] -= h
            fd = (L(p) - L(m)) / (2 * h)
            assert abs(fd - dl[t, e]) <= 1e-8
    # unselected experts get exactly zero; rows sum to zero
    mask = np.ones((T, E), bool)
    np.put_along_axis(mask, ids.astype(np.int64), False, axis=1)
    assert np.all(dl[mask] == 0.0)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-15)
