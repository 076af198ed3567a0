"""GPU parity: every entry point of libgq against the fp64 oracle on the same
seeded inputs (small and ragged shapes that still span several tiles).

Bars: bit-exact for block decode (float32 and bf16) and for the routing
integers; relative Frobenius error <= 1e-2 for every floating-point output
(bf16 inputs and outputs, fp32 accumulation)."""
import sys

import numpy as np
import pytest

import synth
from oracle import adamw8bit as oa
from oracle import blocks as ob
from oracle import linear as ol
from oracle import lmhead as olm
from oracle import moe as om
from oracle import rmsnorm as orms
from oracle import routing as orr

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_base_lora_amd as gq  # noqa: E402
from gpu_helpers import (bf16_dev, check, f32_dev, host, i32_dev, i64_dev, same_f32_bits,  # noqa: E402
                         u8_dev)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------- dequant
def test_dequant_golden(golden_blocks):
    for c in golden_blocks:
        raw = np.frombuffer(c["bytes"], np.uint8).reshape(1, -1)
        say("dequant golden", c["name"])
        got = host(gq.dequant(c["qtype"], u8_dev(raw), 1, 32))[0]
        same_f32_bits(got, np.array(c["expect"], np.float32))


@pytest.mark.parametrize("qtype", [0, 1, 2])
@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (33, 2048), (257, 160)])
def test_dequant_random(qtype, rows, cols):
    rng = np.random.default_rng(rows * 31 + cols + qtype)
    w = (0.02 * rng.standard_normal((rows, cols))).astype(np.float32)
    raw = synth.quantize(qtype, w)
    # scramble some scales into subnormal / negative / zero fp16 values
    bs = synth.BLOCK_BYTES[qtype]
    v = raw.reshape(rows, cols // 32, bs)
    v[0, 0, 0:2] = [0x01, 0x00]
    if rows > 1:
        v[1, -1, 0:2] = [0x00, 0x84]
    say("dequant random", qtype, rows, cols)
    exp = ob.dequant_f32(qtype, raw, rows, cols)
    d = u8_dev(raw)
    same_f32_bits(host(gq.dequant(qtype, d, rows, cols)), exp)
    got16 = gq.dequant(qtype, d, rows, cols, torch.bfloat16)
    exp16 = synth.f32_to_bf16_bits(exp)
    assert np.array_equal(got16.view(torch.int16).cpu().numpy().view(np.uint16), exp16)


# ------------------------------------------------------------------ linear
def lin_proj(inp):
    return gq.Proj(inp["qtype"], inp["N"], inp["K"], u8_dev(inp["blocks"]), f32_dev(inp["A"]),
                   f32_dev(inp["B"]), float(inp["scale"]))


LIN_CASES = [
    (1, 64, 8, 0, 1), (5, 128, 96, 1, 2), (129, 256, 200, 2, 4), (128, 1024, 1024, 0, 4),
    (300, 512, 520, 1, 8), (77, 192, 136, 2, 16),
    # T <= 64, K % 256 == 0: the skinny forward MMQ with 16-, 32- and 64-row
    # tiles, ragged last column tile
    (9, 256, 200, 0, 4), (20, 512, 264, 1, 8), (33, 256, 136, 2, 4), (64, 512, 128, 1, 16),
]


@pytest.mark.parametrize("T,K,N,qtype,r", LIN_CASES)
@pytest.mark.parametrize("large", [False, True])
def test_linear_fwd_bwd(T, K, N, qtype, r, large):
    cfg = synth.LinearCfg("t", T=T, K=K, N=N, qtype=qtype, rank=r, alpha=2.0 * r, seed=T + K)
    inp = synth.make_linear(cfg, large_adapter=large)
    ref = ol.run(inp)
    say("linear", T, K, N, qtype, r, large)
    p = lin_proj(inp)
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])
    y, xa = gq.linear_lora_fwd(p, x)
    dx, dA, dB = gq.linear_lora_bwd(p, x, xa, dy)
    torch.cuda.synchronize()
    check("y", host(y), ref["y"])
    check("xa", host(xa), ref["xa"])
    check("dx", host(dx), ref["dx"])
    check("dA", host(dA), ref["dA"])
    check("dB", host(dB), ref["dB"])


def test_linear_b_zero_is_base_and_da_zero():
    cfg = synth.LinearCfg("t", T=64, K=256, N=128, qtype=1, rank=4, alpha=8)
    inp = synth.make_linear(cfg, large_adapter=True)
    inp["B"][:] = 0.0
    ref = ol.run(inp)
    p = lin_proj(inp)
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])
    y, xa = gq.linear_lora_fwd(p, x)
    dx, dA, dB = gq.linear_lora_bwd(p, x, xa, dy)
    torch.cuda.synchronize()
    check("y", host(y), ref["y"])
    assert np.all(host(dA) == 0.0)
    check("dB", host(dB), ref["dB"])


def test_linear_one_hot_rows_bit_exact():
    """x[t] = e_k and B = 0: y[t] = bf16(deq(W)[:, k]) exactly."""
    cfg = synth.LinearCfg("t", T=8, K=128, N=64, qtype=0, rank=4, alpha=8)
    inp = synth.make_linear(cfg)
    cols = [0, 5, 31, 32, 63, 64, 100, 127]
    X = np.zeros((8, 128), np.float32)
    for t, c in enumerate(cols):
        X[t, c] = 1.0
    inp["x"] = synth.f32_to_bf16_bits(X)
    inp["B"][:] = 0.0
    W = ob.dequant_f32(0, inp["blocks"], 64, 128)
    y, _ = gq.linear_lora_fwd(lin_proj(inp), bf16_dev(inp["x"]))
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    for t, c in enumerate(cols):
        assert np.array_equal(got[t], synth.f32_to_bf16_bits(W[:, c]))


def test_linear_deterministic():
    cfg = synth.LinearCfg("t", T=200, K=512, N=256, qtype=1, rank=4, alpha=8)
    inp = synth.make_linear(cfg, large_adapter=True)
    p = lin_proj(inp)
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])
    outs = []
    for _ in range(2):
        y, xa = gq.linear_lora_fwd(p, x)
        dx, dA, dB = gq.linear_lora_bwd(p, x, xa, dy)
        outs.append([t.clone() for t in (y, xa, dx, dA, dB)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ----------------------------------------------------------------- routing
# T k <= 256 runs the one-block routing kernel, larger counts the chunked one
@pytest.mark.parametrize("T,E,k,zipf", [(37, 8, 2, 0.0), (1000, 128, 8, 0.0), (4096, 256, 8, 1.0),
                                        (5, 1, 1, 0.0), (64, 16, 16, 0.0), (300, 1024, 16, 0.0),
                                        (16, 1024, 16, 1.0), (32, 128, 8, 0.0), (33, 128, 8, 0.0),
                                        (16, 60, 8, 0.0), (100, 200, 8, 1.0), (50, 600, 4, 0.0)])
def test_route_bit_exact(T, E, k, zipf):
    rng = np.random.default_rng(T + E)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if zipf:
        logits = logits + synth.zipf_bias(E, zipf, rng)
    # inject exact ties
    logits[0, : min(E, 4)] = 0.5
    say("route", T, E, k)
    ids, w, s, off, pos = gq.moe_route(f32_dev(logits), k)
    rid, rw, rs, roff, rpos = orr.route(logits, k)
    assert np.array_equal(host(ids), rid)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(off), roff)
    assert np.array_equal(host(pos), rpos)
    check("w", host(w), rw, 1e-5)


def test_route_bwd():
    rng = np.random.default_rng(3)
    T, E, k = 100, 32, 4
    logits = rng.standard_normal((T, E), dtype=np.float32)
    ids, w = orr.topk(logits, k)
    dw = rng.standard_normal((T, k))
    ref = orr.backward(ids, w, dw, E)
    got = gq.moe_route_bwd(i32_dev(ids), f32_dev(w), f32_dev(dw), E)
    check("dlogits", host(got), ref, 1e-5)


# --------------------------------------------------------------------- MoE
def moe_weights(inp):
    E, H, I = inp["E"], inp["H"], inp["I"]
    s = float(inp["scale"])
    qt = inp["qtype"]
    gate = gq.Proj(qt, I, H, u8_dev(inp["wg"]), f32_dev(inp["ag"]), f32_dev(inp["bg"]), s, E)
    up = gq.Proj(qt, I, H, u8_dev(inp["wu"]), f32_dev(inp["au"]), f32_dev(inp["bu"]), s, E)
    down = gq.Proj(qt, H, I, u8_dev(inp["wd"]), f32_dev(inp["ad"]), f32_dev(inp["bd"]), s, E)
    return gq.MoEWeights(gate, up, down)


MOE_CASES = [
    # T, H, I, E, k, qtype, rank, zipf
    (24, 64, 64, 4, 2, 1, 2, 0.0),
    (100, 128, 128, 8, 2, 0, 4, 0.0),
    (257, 256, 192, 16, 4, 2, 8, 1.0),
    (64, 128, 64, 32, 8, 1, 4, 1.0),  # many idle experts
    (200, 128, 64, 100, 4, 1, 4, 0.5),  # E not a multiple of 64: partly filled prefix lanes
    # few rows per expert, K % 256 == 0: the skinny forward MMQ (16-row tiles,
    # 32-row tiles in the last case); in the first only the down projection
    # (K = I = 256) runs skinny, on a ragged last column tile (H = 320)
    (40, 320, 256, 8, 2, 0, 4, 1.0),
    (48, 512, 256, 8, 2, 1, 4, 1.0),
    (30, 256, 256, 4, 2, 2, 8, 0.0),
    (64, 256, 256, 4, 2, 1, 4, 0.5),
    # at most 8 rows per expert: the gate/up backward on the skinny NN MMQ
    (24, 256, 128, 8, 2, 2, 4, 1.0),
    (16, 512, 192, 16, 2, 0, 8, 0.0),
    # ... and with I % 256 == 0 also the down backward (SwiGLU-backward
    # epilogue; rank 16 reads the up/gate B rows from global memory)
    (24, 256, 256, 8, 2, 1, 4, 1.0),
    (20, 512, 512, 16, 2, 0, 8, 0.0),
    (16, 256, 768, 8, 4, 2, 16, 1.0),
]


@pytest.mark.parametrize("T,H,I,E,k,qtype,r,zipf", MOE_CASES)
def test_moe_layer(T, H, I, E, k, qtype, r, zipf):
    cfg = synth.MoECfg("t", T=T, H=H, I=I, E=E, k=k, qtype=qtype, rank=r, alpha=2.0 * r, zipf=zipf,
                       seed=T + E)
    inp = synth.make_moe(cfg, large_adapter=True, w_sigma=0.05)
    say("moe", T, H, I, E, k, qtype, r)
    f = om.forward(inp)
    b = om.backward(inp, f)
    wts = moe_weights(inp)
    x, dy, lg = bf16_dev(inp["x"]), bf16_dev(inp["dy"]), f32_dev(inp["logits"])
    y, saved = gq.moe_ffn_fwd(wts, x, lg, k)
    g = gq.moe_ffn_bwd(wts, x, dy, saved, k, E)
    torch.cuda.synchronize()
    assert np.array_equal(host(saved["ids"]), f["ids"])
    assert np.array_equal(host(saved["sorted"]), f["sorted"])
    assert np.array_equal(host(saved["offsets"]), f["offsets"])
    check("g", host(saved["g"]), f["g"])
    check("u", host(saved["u"]), f["u"])
    check("h", host(saved["h"]), f["h"])
    check("o", host(saved["o"]), f["o"])
    check("y", host(y), f["y"])
    check("dw", host(g["dw"]), b["dw"])
    check("dx", host(g["dx"]), b["dx"])
    check("dlogits", host(g["dlogits"]), b["dlogits"])
    for n in ("dA_d", "dB_d", "dA_g", "dB_g", "dA_u", "dB_u"):
        ref = b[n.replace("_", "")]
        got = host(g[n])
        check(n, got, ref)
        idle = np.diff(f["offsets"]) == 0
        assert np.all(got[idle] == 0.0), f"{n}: idle experts must get exact zeros"


# ----------------------------------------------------------------- LM head
HEAD_CASES = [
    # T, H, V, chunk, qtype, ignore_frac
    (5, 64, 520, 256, 0, 0.0),
    (130, 128, 1000, 384, 1, 0.2),
    (64, 256, 4096, 4096, 2, 0.0),
    (200, 192, 3000, 1024, 0, 0.1),
    # T <= 32 with H % 256 == 0: the skinny logits pass; ragged vocabulary tile
    (16, 256, 1000, 1000, 0, 0.1),
    (30, 512, 3000, 1024, 1, 0.0),
    (7, 256, 712, 712, 2, 0.2),
    # more than 64 tokens and 256 vocabulary tiles: the multi-block merge
    (100, 256, 40000, 16384, 0, 0.1),
]


@pytest.mark.parametrize("T,H,V,chunk,qtype,ign", HEAD_CASES)
def test_lmhead(T, H, V, chunk, qtype, ign):
    cfg = synth.HeadCfg("t", T=T, H=H, V=V, qtype=qtype, rank=4, alpha=8, chunk=chunk,
                        ignore_frac=ign, seed=T + V)
    inp = synth.make_head(cfg, large_adapter=True, w_sigma=0.05)
    say("lmhead", T, H, V, chunk, qtype)
    ref = olm.forward_backward(inp, chunk=chunk)
    head = gq.Proj(qtype, V, H, u8_dev(inp["blocks"]), f32_dev(inp["A"]), f32_dev(inp["B"]),
                   float(inp["scale"]))
    out = gq.lmhead_chunked_ce(head, bf16_dev(inp["h"]), i64_dev(inp["labels"]), chunk_rows=chunk)
    torch.cuda.synchronize()
    assert abs(float(out["loss"]) - ref["loss"]) <= 1e-3 * abs(ref["loss"])
    check("lse", host(out["lse"]), ref["lse"], 1e-4)
    check("dh", host(out["dh"]), ref["dh"])
    check("dA", host(out["dA"]), ref["dA"])
    check("dB", host(out["dB"]), ref["dB"])
    ign_rows = inp["labels"] == -100
    assert np.all(host(out["dh"])[ign_rows] == 0.0)
    assert int(out["ws"][:4].view(torch.int32).item()) == 0


def test_lmhead_bad_label_flag():
    cfg = synth.HeadCfg("t", T=16, H=64, V=256, qtype=0, rank=4, alpha=8, chunk=128)
    inp = synth.make_head(cfg)
    inp["labels"][3] = 999
    head = gq.Proj(0, 256, 64, u8_dev(inp["blocks"]), f32_dev(inp["A"]), f32_dev(inp["B"]),
                   float(inp["scale"]))
    out = gq.lmhead_chunked_ce(head, bf16_dev(inp["h"]), i64_dev(inp["labels"]), chunk_rows=128)
    torch.cuda.synchronize()
    assert int(out["ws"][:4].view(torch.int32).item()) != 0
    inp["labels"][3] = -100
    ref = olm.forward_backward(inp, chunk=128)
    assert abs(float(out["loss"]) - ref["loss"]) <= 1e-3 * ref["loss"]


# ---------------------------------------------------------------- RMSNorm
# H up to 4096 keeps a row in registers, longer rows read x twice
NORM_CASES = [(1, 8, 1e-6), (5, 64, 1e-6), (37, 320, 1e-2), (256, 2048, 1e-6), (64, 4096, 1e-5),
              (33, 4104, 1e-6), (3, 8192, 1e-6)]


@pytest.mark.parametrize("T,H,eps", NORM_CASES)
def test_rmsnorm(T, H, eps):
    rng = np.random.default_rng(T * 7 + H)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= np.exp(rng.uniform(-4, 4, (T, 1))).astype(np.float32)  # rows of very different scale
    if T > 2:
        x[1] = 0.0  # zero row: rstd = 1/sqrt(eps), y = 0
    xb = synth.f32_to_bf16_bits(x)
    w = rng.uniform(0.5, 1.5, H).astype(np.float32)
    dyb = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    xr = synth.bf16_bits_to_f32(xb).astype(np.float64)
    dyr = synth.bf16_bits_to_f32(dyb).astype(np.float64)
    say("rmsnorm", T, H, eps)
    y, rstd = gq.rmsnorm_fwd(bf16_dev(xb), f32_dev(w), eps)
    dx = gq.rmsnorm_bwd(bf16_dev(dyb), bf16_dev(xb), f32_dev(w), rstd)
    torch.cuda.synchronize()
    ref_y, ref_r = orms.forward(xr, w, eps)
    ref_dx = orms.backward(xr, w, dyr, eps)
    check("rstd", host(rstd), ref_r, 1e-5)
    check("y", host(y), ref_y)
    check("dx", host(dx), ref_dx)


def test_rmsnorm_deterministic():
    rng = np.random.default_rng(11)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((100, 2048)).astype(np.float32))
    w = f32_dev(rng.uniform(0.5, 1.5, 2048))
    x = bf16_dev(xb)
    a = gq.rmsnorm_fwd(x, w)
    b = gq.rmsnorm_fwd(x, w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------ 8-bit AdamW
# codes, scales and parameters bit-exact against the oracle over several
# steps (both sides take the same float32 operations in the same order)
@pytest.mark.parametrize("n,steps,wd", [(1, 3, 0.0), (256, 4, 0.01), (700, 5, 0.0), (100003, 3, 0.1)])
def test_adamw8bit_bit_exact(n, steps, wd):
    rng = np.random.default_rng(n + steps)
    p0 = rng.standard_normal(n).astype(np.float32)
    p = torch.from_numpy(p0.copy()).cuda()
    st = gq.AdamW8bitState(n, p.device)
    ph, mq, vq = p0.copy(), np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    nb = (n + 255) // 256
    sm, sv = np.zeros(nb, np.float32), np.zeros(nb, np.float32)
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    say("adamw8bit", n, steps, wd)
    for t in range(1, steps + 1):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 1)).astype(np.float32)
        if t == 2 and n > 300:
            g[256:300] = 0.0  # a stretch of zero gradients
        if n == 700:
            g[512:] *= 1e-20  # the last block's v scale stays below 2^-126
        gq.adamw8bit_step(p, torch.from_numpy(g).cuda(), st, lr, (b1, b2), eps, wd)
        ph, mq, vq, sm, sv = oa.step(ph, g, mq, vq, sm, sv, t, lr, b1, b2, eps, wd)
    torch.cuda.synchronize()
    assert np.array_equal(st.m_codes.cpu().numpy(), mq)
    assert np.array_equal(st.v_codes.cpu().numpy(), vq)
    assert np.array_equal(st.m_scale.cpu().numpy().view(np.uint32), sm.view(np.uint32))
    assert np.array_equal(st.v_scale.cpu().numpy().view(np.uint32), sv.view(np.uint32))
    assert np.array_equal(p.cpu().numpy().view(np.uint32), ph.view(np.uint32))
