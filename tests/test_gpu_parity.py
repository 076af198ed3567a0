"""GPU parity: every entry point of libgq against the fp64 oracle on the same
seeded inputs (small and ragged shapes that still span several tiles).

Bars: bit-exact for block decode (float32 and bf16) and for the routing
integers; relative Frobenius error <= 1e-2 for every floating-point output
(bf16 inputs and outputs, fp32 accumulation)."""
import sys

import numpy as np
import pytest

import synth
from moe_cases import SPILL_CASES
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
from gpu_helpers import (bf16_dev, check, check_per_expert, f32_dev, host, i32_dev, i64_dev,  # noqa: E402
                         same_f32_bits, u8_dev)


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
    # an odd number of blocks per weight row (n_in % 64 == 32): the reduction
    # ends in a half k-step, rows start 2-byte aligned
    (19, 32, 40, 1, 4), (70, 96, 136, 0, 8), (130, 160, 64, 2, 4), (300, 160, 200, 1, 16),
    (257, 96, 264, 0, 2),
    # enough 256 x 192 tiles for the wide forward MMQ, with a partial last
    # row tile and a partial last column tile (T % 256, N % 192 != 0)
    (2000, 1024, 6104, 0, 4), (1800, 512, 5760, 1, 8),
    # few tiles: the reduction split over workgroups, summed by the fixup
    # pass (forward and dX; ragged rows)
    (100, 512, 512, 2, 8), (90, 256, 1024, 1, 4),
    # dY B over four column ranges (unequal, ragged last) summed by the dB / dA
    # reduction
    (700, 256, 4000, 1, 4), (500, 128, 3200, 0, 16),
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


@pytest.mark.parametrize("qtype", [0, 1, 2])
@pytest.mark.parametrize("T,K,N", [(8, 128, 64), (16, 256, 128), (300, 512, 384)])
def test_linear_one_hot_rows_bit_exact(qtype, T, K, N):
    """One-hot rows with B = 0 read single decoded weights back exactly:
    x[t] = e_k gives y[t] = bf16(deq(W)[:, k]) (forward, the weight tile's
    decode along its rows), dY[t] = e_n gives dX[t] = bf16(deq(W)[n, :])
    (backward, the decode of whole weight rows)."""
    cfg = synth.LinearCfg("t", T=T, K=K, N=N, qtype=qtype, rank=4, alpha=8, seed=T + qtype)
    inp = synth.make_linear(cfg)
    rng = np.random.default_rng(T + 7 * qtype)
    cols = rng.integers(0, K, T)
    rows = rng.integers(0, N, T)
    cols[:4] = [0, 31, 32, K - 1]
    rows[:4] = [0, 31, 32, N - 1]
    X = np.zeros((T, K), np.float32)
    X[np.arange(T), cols] = 1.0
    DY = np.zeros((T, N), np.float32)
    DY[np.arange(T), rows] = 1.0
    inp["x"] = synth.f32_to_bf16_bits(X)
    inp["dy"] = synth.f32_to_bf16_bits(DY)
    inp["B"][:] = 0.0
    W = ob.dequant_f32(qtype, inp["blocks"], N, K)
    say("one-hot", qtype, T, K, N)
    p = lin_proj(inp)
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])
    y, xa = gq.linear_lora_fwd(p, x)
    dx, _, _ = gq.linear_lora_bwd(p, x, xa, dy)
    # bits compared with -0 read as +0: the fused decode forms d*(q - z) as
    # d*q' + (-z*d), whose exact zero is +0 where d*0 is -0 for d < 0
    def bits(a):
        a = np.asarray(a, np.uint16).copy()
        a[(a & 0x7FFF) == 0] = 0
        return a
    gy = y.view(torch.int16).cpu().numpy().view(np.uint16)
    gdx = dx.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits(gy), bits(synth.f32_to_bf16_bits(W[:, cols].T))), "forward"
    assert np.array_equal(bits(gdx), bits(synth.f32_to_bf16_bits(W[rows, :]))), "backward"


@pytest.mark.parametrize("qtype", [0, 1, 2])
def test_linear_nonfinite_scales(qtype):
    """Blocks with an infinite or NaN scale: inside the MMQ the outputs they
    feed are non-finite exactly where the oracle's are (the fused decode may
    give NaN where d*q is +-inf, so only finiteness is compared there); every
    other output meets the usual bar."""
    cfg = synth.LinearCfg("nf", T=40, K=128, N=64, qtype=qtype, rank=4, alpha=8)
    inp = synth.make_linear(cfg, large_adapter=True)
    bs = synth.BLOCK_BYTES[qtype]
    v = inp["blocks"].reshape(cfg.N, cfg.K // 32, bs)
    v[5, 1, 0:2] = [0x00, 0x7C]   # +inf
    v[20, 0, 0:2] = [0x00, 0xFC]  # -inf
    v[33, 3, 0:2] = [0x00, 0x7E]  # NaN
    say("linear non-finite scales", qtype)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = ol.run(inp)
    p = lin_proj(inp)
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])
    y, xa = gq.linear_lora_fwd(p, x)
    dx, dA, dB = gq.linear_lora_bwd(p, x, xa, dy)
    torch.cuda.synchronize()
    for n, got in (("y", y), ("dx", dx)):
        g = host(got)
        fin = np.isfinite(ref[n])
        assert (~fin).any(), n
        assert np.array_equal(np.isfinite(g), fin), f"{n}: non-finite pattern differs"
        e = np.linalg.norm(g[fin] - ref[n][fin]) / np.linalg.norm(ref[n][fin])
        assert e <= 1e-2, (n, e)
    check("dA", host(dA), ref["dA"])
    check("dB", host(dB), ref["dB"])


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
                                        (16, 60, 8, 0.0), (100, 200, 8, 1.0), (50, 600, 4, 0.0),
                                        (128, 128, 8, 1.0), (205, 64, 5, 0.0), (128, 3, 3, 0.0)])
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
    # hidden size with an odd number of blocks (H % 64 == 32)
    (60, 96, 64, 4, 2, 1, 4, 0.0),
    (150, 160, 128, 8, 2, 0, 8, 1.0),
] + SPILL_CASES


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
    check("dg", host(g["dg"]), b["dg"])
    check("du", host(g["du"]), b["du"])
    check("dx", host(g["dx"]), b["dx"])
    check("dlogits", host(g["dlogits"]), b["dlogits"])
    idle = np.diff(f["offsets"]) == 0
    for n in ("dA_d", "dB_d", "dA_g", "dB_g", "dA_u", "dB_u"):
        ref = b[n.replace("_", "")]
        got = host(g[n])
        check(n, got, ref)
        check_per_expert(n, got, ref, np.diff(f["offsets"]))  # every active expert on its own, exact zeros for idle ones
        assert np.all(got[idle] == 0.0), f"{n}: idle experts must get exact zeros"


@pytest.mark.parametrize("T,qtype", [(40, 1), (300, 0), (24, 2)])
def test_idle_experts_blocks_unused(T, qtype):
    """Only experts that own rows touch their blocks: every idle expert's
    blocks get NaN scales, and the whole layer (forward and backward) must
    give bitwise the same results as with clean blocks.  (The counter side,
    that those blocks are not even fetched, is the grouped-launch FETCH_SIZE
    profile.)"""
    E, k, H, I, r = 16, 2, 128, 128, 4
    cfg = synth.MoECfg("t", T=T, H=H, I=I, E=E, k=k, qtype=qtype, rank=r, alpha=8, seed=T)
    inp = synth.make_moe(cfg, large_adapter=True)
    active = [1, 6, 7, 12]
    idle = [e for e in range(E) if e not in active]
    inp["logits"][:, idle] = -1e4  # never among the top k
    say("idle experts", T, qtype, "active", active)
    runs = []
    for poison in (False, True):
        bl = {n: np.array(inp[n], copy=True) for n in ("wg", "wu", "wd")}
        if poison:
            for n in bl:
                blocks = bl[n].reshape(E, -1, synth.BLOCK_BYTES[qtype])
                blocks[idle, :, 0] = 0x00  # fp16 scale d = NaN (0x7E00)
                blocks[idle, :, 1] = 0x7E
                if qtype == 2:
                    blocks[idle, :, 2] = 0x00  # and min m = NaN
                    blocks[idle, :, 3] = 0x7E
        s = float(inp["scale"])
        wts = gq.MoEWeights(gq.Proj(qtype, I, H, u8_dev(bl["wg"]), f32_dev(inp["ag"]), f32_dev(inp["bg"]), s, E),
                            gq.Proj(qtype, I, H, u8_dev(bl["wu"]), f32_dev(inp["au"]), f32_dev(inp["bu"]), s, E),
                            gq.Proj(qtype, H, I, u8_dev(bl["wd"]), f32_dev(inp["ad"]), f32_dev(inp["bd"]), s, E))
        x, dy, lg = bf16_dev(inp["x"]), bf16_dev(inp["dy"]), f32_dev(inp["logits"])
        y, saved = gq.moe_ffn_fwd(wts, x, lg, k)
        g = gq.moe_ffn_bwd(wts, x, dy, saved, k, E)
        torch.cuda.synchronize()
        offs = host(saved["offsets"])
        assert set(np.flatnonzero(np.diff(offs))) == set(active)
        out = {"y": y, "h": saved["h"], "o": saved["o"]}
        out.update({n: g[n] for n in ("dx", "dlogits", "dw", "dg", "du", "dA_d", "dB_d", "dA_g", "dB_g",
                                      "dA_u", "dB_u")})
        runs.append({n: host(t) for n, t in out.items()})
    clean, poisoned = runs
    for n in clean:
        assert np.isfinite(clean[n]).all(), n
        say("bitwise equal:", n)
        same_f32_bits(np.asarray(poisoned[n], np.float32), np.asarray(clean[n], np.float32))


def test_grouped_offsets_checked_on_device():
    """Inconsistent expert offsets (decreasing, not ending at M) set the
    workspace's error word and no row is processed; consistent offsets on
    the same workspace clear it."""
    cfg = synth.MoECfg("t", T=32, H=128, I=64, E=4, k=2, qtype=1, rank=4, alpha=8)
    inp = synth.make_moe(cfg)
    wts = moe_weights(inp)
    x = bf16_dev(inp["x"])
    M = cfg.T * cfg.k
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    gather = torch.arange(M, dtype=torch.int32, device="cuda")
    for offs, bad in (([0, 30, 20, 50, M], True), ([0, 10, 20, 30, M - 4], True), ([4, 10, 20, 30, M], True),
                      ([0, 10, 20, 30, M], False)):
        say("offsets", offs)
        gq.grouped_mmq_lora_fwd([wts.gate, wts.up], gq.EPI_SWIGLU, x, gather, cfg.k,
                                i32_dev(np.array(offs)), M, ws=ws)
        torch.cuda.synchronize()
        word = int(ws[:4].view(torch.int32).item())
        assert (word != 0) == bad, (offs, word)


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
    # hidden size with an odd number of blocks; vocabulary sizes that are not
    # a multiple of 8 (tile and skinny logits passes)
    (40, 96, 701, 256, 1, 0.1),
    (150, 160, 2000, 512, 0, 0.0),
    (16, 256, 1001, 333, 2, 0.1),
    # enough 256 x 192 tiles for the wide logits pass (ragged rows and
    # vocabulary tile)
    (600, 128, 30000, 8192, 1, 0.1),
    (720, 64, 26000, 26000, 0, 0.0),
    # 128-row tiles over several chunks (gradient tiles of a chunk share a
    # launch with the previous chunk's dh tiles), last chunk of 6 rows,
    # hidden size with an odd number of blocks
    (768, 96, 16390, 4096, 0, 0.2),
]


# 256 x 192 gradient tiles over several chunks per launch, ranks taken four
# at a time in their epilogue (rank 8, 6 and 12; ragged rows, ragged last
# step, one k-step of hidden size); the dh sums on 256 x 128 tiles over two
# steps (ragged rows and reduction, a half-used column tile) or one
HEAD_WIDE_RANK_CASES = [
    # T, H, V, chunk, qtype, ignore_frac, rank
    (768, 128, 20000, 2048, 0, 0.1, 8),
    (600, 64, 14000, 2048, 1, 0.0, 6),
    (1024, 64, 10000, 4096, 1, 0.2, 12),
    (600, 192, 14000, 2048, 0, 0.1, 4),
    # last step of 12 vocabulary rows: one ragged k-step, the first dh range
    # of that step empty
    (768, 128, 12300, 2048, 1, 0.1, 4),
]


@pytest.mark.parametrize("T,H,V,chunk,qtype,ign", HEAD_CASES)
def test_lmhead(T, H, V, chunk, qtype, ign):
    _lmhead_case(T, H, V, chunk, qtype, ign, 4)


@pytest.mark.parametrize("T,H,V,chunk,qtype,ign,rank", HEAD_WIDE_RANK_CASES)
def test_lmhead_wide_ranks(T, H, V, chunk, qtype, ign, rank):
    _lmhead_case(T, H, V, chunk, qtype, ign, rank)


def _lmhead_case(T, H, V, chunk, qtype, ign, rank):
    cfg = synth.HeadCfg("t", T=T, H=H, V=V, qtype=qtype, rank=rank, alpha=2 * rank, chunk=chunk,
                        ignore_frac=ign, seed=T + V)
    inp = synth.make_head(cfg, large_adapter=True, w_sigma=0.05)
    say("lmhead", T, H, V, chunk, qtype, rank)
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
    # every row of G sums to 0, so the columns of dB = s G^T xa sum to 0
    # (the reference is 0 in exact arithmetic: compare against the size of dB)
    dB = host(out["dB"]).astype(np.float64)
    assert np.all(np.abs(dB.sum(axis=0)) <= 1e-3 * np.abs(dB).sum(axis=0) + 1e-30)


def test_lmhead_all_labels_ignored():
    """No valid label: loss 0 and every gradient exactly 0, lse still the
    log-sum-exp of the logits."""
    cfg = synth.HeadCfg("t", T=40, H=128, V=900, qtype=1, rank=4, alpha=8, chunk=256)
    inp = synth.make_head(cfg, large_adapter=True)
    inp["labels"][:] = -100
    ref = olm.forward_backward(inp, chunk=256)
    head = gq.Proj(1, 900, 128, u8_dev(inp["blocks"]), f32_dev(inp["A"]), f32_dev(inp["B"]),
                   float(inp["scale"]))
    out = gq.lmhead_chunked_ce(head, bf16_dev(inp["h"]), i64_dev(inp["labels"]), chunk_rows=256)
    torch.cuda.synchronize()
    assert float(out["loss"]) == 0.0 and ref["loss"] == 0.0
    check("lse", host(out["lse"]), ref["lse"], 1e-4)
    for n in ("dh", "dA", "dB"):
        assert np.all(host(out[n]) == 0.0), n
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
U32 = 2.0 ** -24  # unit roundoff of float32


def adamw_check_step(ref, p_gpu, mq, vq, sm, sv):
    """Validity of one GPU step against the float64 oracle step taken from
    the same stored state.  The kernel works in float32; the bounds below
    follow from a bounded number of float32 roundings per quantity (u =
    2^-24), with a factor of two to spare:
      m' has <= 4 roundings of terms of size Cm = |b1 m| + |(1 - b1) g|;
      v' <= 6 roundings of positive terms; the block scale is the largest
      of these; a normalised state x/scale picks up the error of x over the
      scale, its own size times the scale's relative error, and 3 roundings
      of its own;
      p' = p - lr (mhat / (sqrt(vhat) + eps) + wd p): 3 roundings at the
      size of p, 10 at the size of the update, 4 Cm at the size of m'.
    Below 2^-126 a float32 rounding errs by up to 2^-150 absolute (the
    subnormal spacing), which the scale bound allows for.
    Codes must be the nearest book entry, except where the exact
    normalised state lies within its error bound of the midpoint between
    two neighbouring entries: there either neighbour is accepted.  Returns
    the number of such elements."""
    n = p_gpu.size
    b1, lr, wd, t, eps = ref["b1"], ref["lr"], ref["wd"], ref["t"], ref["eps"]
    cm = np.abs(b1 * ref["m_in"]) + np.abs((1 - b1) * ref["g"])
    # p
    mhat = np.abs(ref["m"]) / (1 - b1 ** t)
    den = np.sqrt(ref["v"] / (1 - ref["b2"] ** t)) + eps
    p_in = ref["p_in"]
    bound_p = 2 * (3 * U32 * np.abs(p_in) + U32 * np.abs(ref["p"]) +
                   lr * (10 * U32 * mhat + 4 * U32 * cm / (1 - b1 ** t)) / den)
    err_p = np.abs(p_gpu.astype(np.float64) - ref["p"])
    assert np.all(err_p <= bound_p), f"p: {np.sum(err_p > bound_p)} outside the float32 bound"
    band = 0
    for state, codes, scale, table, c_el in (("m", mq, sm, oa.signed_table(), cm),
                                             ("v", vq, sv, oa.unsigned_table(), np.abs(ref["v"]))):
        exact_scale = ref["scale_" + state]
        nb = exact_scale.size
        cmax = np.array([c_el[256 * b:256 * (b + 1)].max() for b in range(nb)])
        slack = 8 * U32 * cmax + 8 * 2.0 ** -149  # float32 subnormals round at an absolute 2^-150
        err_s = np.abs(scale.astype(np.float64) - exact_scale)
        assert np.all(err_s <= 1e-6 * exact_scale + slack), f"{state} scales outside 1e-6"
        xn = ref[state + "n"]
        s_el = np.repeat(np.maximum(exact_scale, 1e-300), 256)[:n]
        tol = 8 * U32 * c_el / s_el + np.abs(xn) * (8 * U32 * np.repeat(cmax, 256)[:n] / s_el + 6 * U32)
        tiny = np.repeat(exact_scale < oa.TINY, 256)[:n]
        want = oa.quantize(xn, table)
        lo, hi, dmid = oa.neighbours(xn, table)
        amb = (dmid <= tol) & (lo != hi) & ~tiny
        got_v, want_v = table[codes.astype(np.int64)], table[want.astype(np.int64)]
        ok = (got_v == want_v) | (amb & ((codes == lo) | (codes == hi)))
        assert np.all(ok), f"{state} codes: {np.sum(~ok)} not the nearest entry"
        assert np.all(codes[tiny] % 128 == 0), f"{state}: a block below 2^-126 must store code 0"
        band += int(amb.sum())
    return band


# every step checked against the float64 oracle step taken from the GPU's own
# state before it (p within float32 bounds, scales within 1e-6, codes the
# nearest entry or, near a midpoint, either neighbour); the chain of steps is
# then checked against the unquantised float64 AdamW
@pytest.mark.parametrize("n,steps,wd", [(1, 3, 0.0), (256, 4, 0.01), (700, 5, 0.0), (100003, 3, 0.1)])
def test_adamw8bit_against_oracle(n, steps, wd):
    rng = np.random.default_rng(n + steps)
    p0 = rng.standard_normal(n).astype(np.float32)
    p = torch.from_numpy(p0.copy()).cuda()
    st = gq.AdamW8bitState(n, p.device)
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    p64 = p0.astype(np.float64)
    m64 = np.zeros(n)
    v64 = np.zeros(n)
    say("adamw8bit", n, steps, wd)
    band = 0
    for t in range(1, steps + 1):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 1)).astype(np.float32)
        if t == 2 and n > 300:
            g[256:300] = 0.0  # a stretch of zero gradients
        if n == 700:
            g[512:] *= 1e-20  # the last block's v scale stays below 2^-126
        before = [a.cpu().numpy() for a in (p, st.m_codes, st.v_codes, st.m_scale, st.v_scale)]
        ref = oa.step_exact(*before[:1], g, *before[1:], t, lr, b1, b2, eps, wd)
        gq.adamw8bit_step(p, torch.from_numpy(g).cuda(), st, lr, (b1, b2), eps, wd)
        torch.cuda.synchronize()
        band += adamw_check_step(ref, p.cpu().numpy(), st.m_codes.cpu().numpy(), st.v_codes.cpu().numpy(),
                                 st.m_scale.cpu().numpy(), st.v_scale.cpu().numpy())
        # unquantised float64 AdamW on the same gradients
        f = lambda x: float(np.float32(x))
        m64 = f(b1) * m64 + (1 - f(b1)) * g
        v64 = f(b2) * v64 + (1 - f(b2)) * g.astype(np.float64) ** 2
        p64 = p64 - f(lr) * (m64 / (1 - f(b1) ** t) / (np.sqrt(v64 / (1 - f(b2) ** t)) + f(eps)) + f(wd) * p64)
    say(f"  {band} codes within float32 error of a midpoint (either neighbour accepted)")
    # the 8-bit states perturb each step's direction by a few per cent of lr
    assert np.max(np.abs(p.cpu().numpy() - p64)) < 0.1 * steps * lr


# Kernel regression (not parity): the float32 model in tests/ repeats the
# kernel's own operations in its order, so codes, scales and p agree bit for
# bit unless the kernel's arithmetic changed.
@pytest.mark.parametrize("n,steps,wd", [(256, 4, 0.01), (700, 5, 0.0)])
def test_adamw8bit_kernel_regression(n, steps, wd):
    import adamw8bit_f32_model as km

    rng = np.random.default_rng(n + steps)
    p0 = rng.standard_normal(n).astype(np.float32)
    p = torch.from_numpy(p0.copy()).cuda()
    st = gq.AdamW8bitState(n, p.device)
    ph, mq, vq = p0.copy(), np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    nb = (n + 255) // 256
    sm, sv = np.zeros(nb, np.float32), np.zeros(nb, np.float32)
    lr, b1, b2, eps = 1e-3, 0.9, 0.999, 1e-8
    for t in range(1, steps + 1):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 1)).astype(np.float32)
        gq.adamw8bit_step(p, torch.from_numpy(g).cuda(), st, lr, (b1, b2), eps, wd)
        ph, mq, vq, sm, sv = km.step(ph, g, mq, vq, sm, sv, t, lr, b1, b2, eps, wd)
    torch.cuda.synchronize()
    assert np.array_equal(st.m_codes.cpu().numpy(), mq)
    assert np.array_equal(st.v_codes.cpu().numpy(), vq)
    assert np.array_equal(st.m_scale.cpu().numpy().view(np.uint32), sm.view(np.uint32))
    assert np.array_equal(st.v_scale.cpu().numpy().view(np.uint32), sv.view(np.uint32))
    assert np.array_equal(p.cpu().numpy().view(np.uint32), ph.view(np.uint32))


# ------------------------------------------------------------ binding checks
def test_binding_rejects_mismatched_tensors_before_launch():
    inp = synth.make_linear(synth.LinearCfg("chk", T=8, K=128, N=64, qtype=synth.Q4_0, rank=4, alpha=8))
    p = lin_proj(inp)
    x = bf16_dev(inp["x"])
    with pytest.raises(TypeError, match="dtype"):
        gq.linear_lora_fwd(p, x.float())
    with pytest.raises(ValueError, match="shape"):
        gq.linear_lora_fwd(p, x[:, :64].contiguous())
    with pytest.raises(ValueError, match="contiguous"):
        gq.linear_lora_fwd(p, torch.cat([x, x], 1)[:, ::2])
    y, xa = gq.linear_lora_fwd(p, x)
    dy = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="xa"):
        gq.linear_lora_bwd(p, x, xa[:4].contiguous(), dy)
    with pytest.raises(ValueError, match="dy"):
        gq.linear_lora_bwd(p, x, xa, dy[:, :32].contiguous())
    short = gq.Proj(p.qtype, p.n_out, p.n_in, p.blocks[:-18], p.A, p.B, p.scale)
    with pytest.raises(ValueError, match="blocks"):
        gq.linear_lora_fwd(short, x)
    with pytest.raises(TypeError, match="labels"):
        gq.lmhead_chunked_ce(p, x, torch.zeros(8, dtype=torch.int32, device="cuda"))
