"""GPU parity at the five full workload sizes, in the launch configuration
bench.py times.

* linear Q8_0 (T 128, 1024 -> 1024) and Q4_0 (T 2048, 2048 -> 6144): every
  output against the full fp64 oracle, both adapter readings.
* MoE Q4_0 (T 2048, H 2048, 128 experts top-8, I 768): every output against
  the full grouped oracle.
* MoE 2-bit, Zipf-skewed (T 4096, H 4096, 256 experts top-8, I 1024, r 8),
  and the Q4_0 MoE weights at T 16 and T 512 (the small-token sweep):
  routing bit-exact; every output as a whole tensor (y, dX, dlogits, dw,
  g, u, h, dg, du and the six adapter gradients) against the oracle run
  one expert at a time (each expert's weights decoded, used and dropped,
  experts spread over host threads), and every active expert's adapter
  gradients on their own.
* LM head Q8_0 (T 2048, H 2048, V 151936, 4096-row chunks), also at T 16
  and T 32: loss, lse, dh, dA, dB against the full chunked oracle.
"""
import dataclasses
import sys

import numpy as np
import pytest

import synth
from oracle import linear as ol
from oracle import lmhead as olm
from oracle import moe as om
from oracle import routing as orr

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_base_lora_amd as gq  # noqa: E402
from gpu_helpers import bf16_dev, check, check_per_expert, f32_dev, host, i64_dev, u8_dev  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfg", [synth.LINEAR_Q8_0_T128, synth.LINEAR_Q4_0_T2048], ids=lambda c: c.name)
@pytest.mark.parametrize("large", [False, True])
def test_linear_full(cfg, large):
    say("fullsize linear", cfg.name, "large" if large else "sigma")
    inp = synth.make_linear(cfg, large_adapter=large)
    ref = ol.run(inp)
    p = gq.Proj(cfg.qtype, cfg.N, cfg.K, u8_dev(inp["blocks"]), f32_dev(inp["A"]),
                f32_dev(inp["B"]), float(inp["scale"]))
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])
    y, xa = gq.linear_lora_fwd(p, x)
    dx, dA, dB = gq.linear_lora_bwd(p, x, xa, dy)
    torch.cuda.synchronize()
    for n, got in (("y", y), ("xa", xa), ("dx", dx), ("dA", dA), ("dB", dB)):
        say(f"  {n}: {check(n, host(got), ref[n]):.2e}")


def _moe_weights(inp):
    E, H, I, s, qt = inp["E"], inp["H"], inp["I"], float(inp["scale"]), inp["qtype"]
    mk = lambda w, a, b, no, ni: gq.Proj(qt, no, ni, u8_dev(w), f32_dev(a), f32_dev(b), s, E)
    return gq.MoEWeights(mk(inp["wg"], inp["ag"], inp["bg"], I, H),
                         mk(inp["wu"], inp["au"], inp["bu"], I, H),
                         mk(inp["wd"], inp["ad"], inp["bd"], H, I))


def test_moe_q4_0_full():
    cfg = synth.MOE_Q4_0_T2048
    say("fullsize moe", cfg.name)
    inp = synth.make_moe(cfg)
    wts = _moe_weights(inp)
    x, dy, lg = bf16_dev(inp["x"]), bf16_dev(inp["dy"]), f32_dev(inp["logits"])
    y, saved = gq.moe_ffn_fwd(wts, x, lg, cfg.k)
    g = gq.moe_ffn_bwd(wts, x, dy, saved, cfg.k, cfg.E)
    torch.cuda.synchronize()
    f = om.forward(inp)
    b = om.backward(inp, f)
    assert np.array_equal(host(saved["ids"]), f["ids"])
    assert np.array_equal(host(saved["sorted"]), f["sorted"])
    assert np.array_equal(host(saved["offsets"]), f["offsets"])
    assert np.array_equal(host(saved["pos"]), f["pos"])
    say(f"  y: {check('y', host(y), f['y']):.2e}")
    for n in ("dx", "dlogits", "dw"):
        say(f"  {n}: {check(n, host(g[n]), b[n]):.2e}")
    for n in ("dg", "du"):
        say(f"  {n}: {check(n, host(g[n]), b[n]):.2e}")
    for n in ("dA_d", "dB_d", "dA_g", "dB_g", "dA_u", "dB_u"):
        ref = b[n.replace('_', '')]
        say(f"  {n}: {check(n, host(g[n]), ref):.2e}, worst expert "
            f"{check_per_expert(n, host(g[n]), ref, np.diff(f['offsets'])):.2f} of its bar")


# the 2-bit workload, and the small-token sweep of the Q4_0 MoE workload at
# its smallest and largest token counts (skinny forward MMQ, 16- and 32-row
# tiles)
SAMPLED_MOE = [
    synth.MOE_Q2DM_T4096_ZIPF,
    dataclasses.replace(synth.MOE_Q4_0_T2048, name="moe_q4_0_t16_h2048_e128k8_i768_r4", T=16),
    dataclasses.replace(synth.MOE_Q4_0_T2048, name="moe_q4_0_t512_h2048_e128k8_i768_r4", T=512),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", SAMPLED_MOE, ids=lambda c: c.name)
def test_moe_expert_by_expert(cfg):
    """Whole-tensor parity with the oracle taken one expert at a time (the
    2-bit workload's 256 experts would need 25 GB as float64 weights)."""
    from concurrent.futures import ThreadPoolExecutor

    say("fullsize moe", cfg.name)
    inp = synth.make_moe(cfg)
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    wts = _moe_weights(inp)
    x, dy, lg = bf16_dev(inp["x"]), bf16_dev(inp["dy"]), f32_dev(inp["logits"])
    y, saved = gq.moe_ffn_fwd(wts, x, lg, k)
    g = gq.moe_ffn_bwd(wts, x, dy, saved, k, E)
    torch.cuda.synchronize()
    ids, w, sorted_, offsets, pos = orr.route(inp["logits"], k)
    assert np.array_equal(host(saved["ids"]), ids)
    assert np.array_equal(host(saved["sorted"]), sorted_)
    assert np.array_equal(host(saved["offsets"]), offsets)
    assert np.array_equal(host(saved["pos"]), pos)
    counts = np.diff(offsets)
    active = [int(e) for e in np.nonzero(counts)[0]]
    say(f"  experts active {len(active)}/{E}, max rows {counts.max()}, median {np.median(counts)}")
    M = T * k
    wflat = w.ravel()
    o = np.zeros((M, H))
    dxrows = np.zeros((M, H))
    dw_flat = np.zeros(M)
    rows = {n: np.zeros((M, I)) for n in ("g", "u", "h", "dg", "du")}
    grads = {n: np.zeros(shape) for n, shape in (
        ("dAd", (E, cfg.rank, I)), ("dBd", (E, H, cfg.rank)), ("dAg", (E, cfg.rank, H)),
        ("dBg", (E, I, cfg.rank)), ("dAu", (E, cfg.rank, H)), ("dBu", (E, I, cfg.rank)))}

    def one(e):
        ew = om.ExpertWeights(inp)
        p0, p1 = offsets[e], offsets[e + 1]
        a = sorted_[p0:p1]
        r = om.expert_backward_rows(inp, e, a, wflat[a], ew)
        ew.drop(e)
        return e, p0, p1, r

    from threadpoolctl import threadpool_limits

    done = 0
    with threadpool_limits(limits=2), ThreadPoolExecutor(8) as ex:
        for e, p0, p1, r in ex.map(one, active):
            o[p0:p1] = r["y_rows"]
            dxrows[p0:p1] = r["dxrows"]
            dw_flat[sorted_[p0:p1]] = r["dw"]
            for n in rows:
                rows[n][p0:p1] = r[n]
            for n in grads:
                grads[n][e] = r[n]
            done += 1
            if done % 32 == 0:
                say(f"  oracle experts {done}/{len(active)}")
    ref_y = np.zeros((T, H))
    ref_dx = np.zeros((T, H))
    for j in range(k):
        a = np.arange(T) * k + j
        ref_y += wflat[a][:, None] * o[pos[a]]
        ref_dx += dxrows[pos[a]]
    dw = dw_flat.reshape(T, k)
    ref_dl = orr.backward(ids, w, dw, E)
    say(f"  y: {check('y', host(y), ref_y):.2e}")
    say(f"  dx: {check('dx', host(g['dx']), ref_dx):.2e}")
    say(f"  dlogits: {check('dlogits', host(g['dlogits']), ref_dl):.2e}")
    say(f"  dw: {check('dw', host(g['dw']), dw):.2e}")
    for n in ("g", "u", "h"):
        say(f"  {n}: {check(n, host(saved[n]), rows[n]):.2e}")
    for n in ("dg", "du"):
        say(f"  {n}: {check(n, host(g[n]), rows[n]):.2e}")
    for n in ("dA_d", "dB_d", "dA_g", "dB_g", "dA_u", "dB_u"):
        got, ref = host(g[n]), grads[n.replace("_", "")]
        say(f"  {n}: {check(n, got, ref):.2e}, worst expert {check_per_expert(n, got, ref, counts):.2f} of its bar")
        assert np.all(got[counts == 0] == 0.0), n


HEAD_FULL = [
    synth.LMHEAD_Q8_0_T2048,
    dataclasses.replace(synth.LMHEAD_Q8_0_T2048, name="lmhead_q8_0_t16_h2048_v151936_r4", T=16),
    dataclasses.replace(synth.LMHEAD_Q8_0_T2048, name="lmhead_q8_0_t32_h2048_v151936_r4", T=32),
]


@pytest.mark.parametrize("cfg", HEAD_FULL, ids=lambda c: c.name)
def test_lmhead_full(cfg):
    say("fullsize lmhead", cfg.name)
    inp = synth.make_head(cfg)
    head = gq.Proj(cfg.qtype, cfg.V, cfg.H, u8_dev(inp["blocks"]), f32_dev(inp["A"]),
                   f32_dev(inp["B"]), float(inp["scale"]))
    out = gq.lmhead_chunked_ce(head, bf16_dev(inp["h"]), i64_dev(inp["labels"]),
                               chunk_rows=cfg.chunk)
    torch.cuda.synchronize()
    ref = olm.forward_backward(inp, chunk=cfg.chunk)
    rel = abs(float(out["loss"]) - ref["loss"]) / ref["loss"]
    say(f"  loss gpu {float(out['loss']):.6f} oracle {ref['loss']:.6f} rel {rel:.2e}")
    assert rel <= 1e-3
    for n, tol in (("lse", 1e-4), ("dh", 1e-2), ("dA", 1e-2), ("dB", 1e-2)):
        say(f"  {n}: {check(n, host(out[n]), ref[n], tol):.2e}")
    assert int(out["ws"][:4].view(torch.int32).item()) == 0
    # rows of G sum to 0: the vocabulary sums of dB vanish up to rounding
    dB = host(out["dB"]).astype(np.float64)
    assert np.all(np.abs(dB.sum(axis=0)) <= 1e-3 * np.abs(dB).sum(axis=0))
