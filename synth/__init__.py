"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This module produces *inputs only*: random draws, the bf16 cast of activations
and the block quantisers that turn fp32 weights into the GGUF-style block bytes
the method reads.  It holds none of the method's arithmetic (no dequantisation,
no matmul, no routing, no loss); the oracle and the HIP path each implement
that on their own.

The pages ("Show HN: LoRA over GGUF - Train Qwen3.8-Flash-Next in 40G VRAM",
section "Things involved in the training") train LoRA adapters on a frozen GGUF
block-quantised base.  The synthetic workloads below follow the shapes the
pages' Qwen3.6-35B-A3B run uses (batch 1, context chunk 2048, LoRA rank 4,
128 experts with 8 active; ai-manual.ru article, the passages on the fused
MoE kernel and the Strix Halo timing) and the five configurations of the
benchmark definition shipped with this project.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# quant type ids (mirrors include/gq.h; plain integers, no arithmetic)
# ---------------------------------------------------------------------------
Q8_0 = 0
Q4_0 = 1
Q2_DM = 2
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q2_DM: 12}
QNAMES = {Q8_0: "q8_0", Q4_0: "q4_0", Q2_DM: "q2_dm"}
QK = 32  # elements per block


# ---------------------------------------------------------------------------
# bf16 input cast (round to nearest even), the dtype activations arrive in
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even, NaN kept."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    out = ((u + r) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# block quantisers (test-data producers).  Each returns uint8 [rows, cols/32*bs]
# ---------------------------------------------------------------------------
def _round_half_away(v: np.ndarray) -> np.ndarray:
    return np.sign(v) * np.floor(np.abs(v) + np.float32(0.5))


def _f16_bytes(d32: np.ndarray) -> np.ndarray:
    """fp32 scales -> little-endian fp16 bytes [..., 2] (RNE via numpy)."""
    return np.ascontiguousarray(d32.astype(np.float16)).view(np.uint8).reshape(*d32.shape, 2)


def quantize_q8_0(w: np.ndarray) -> np.ndarray:
    """Q8_0 blocks: fp16 d = amax/127, int8 q = round(w/d)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % QK == 0
    b = w.reshape(rows, cols // QK, QK)
    amax = np.abs(b).max(axis=2)
    d32 = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(d32 > 0, np.float32(1.0) / d32, np.float32(0.0)).astype(np.float32)
    q = np.clip(_round_half_away(b * inv[..., None]), -127, 127).astype(np.int8)
    out = np.empty((rows, cols // QK, 34), np.uint8)
    out[..., 0:2] = _f16_bytes(d32)
    out[..., 2:] = q.view(np.uint8)
    return out.reshape(rows, -1)


def quantize_q4_0(w: np.ndarray) -> np.ndarray:
    """Q4_0 blocks: d = (signed absmax)/-8, q = clamp(floor(w/d + 8.5), 0, 15).

    Byte j of the 16 payload bytes holds element j in its low nibble and
    element j+16 in its high nibble (GGUF's order)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % QK == 0
    b = w.reshape(rows, cols // QK, QK)
    idx = np.abs(b).argmax(axis=2)  # first index on ties
    mx = np.take_along_axis(b, idx[..., None], axis=2)[..., 0]
    d32 = (mx / np.float32(-8.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(d32 != 0, np.float32(1.0) / d32, np.float32(0.0)).astype(np.float32)
    q = np.clip(np.floor(b * inv[..., None] + np.float32(8.5)), 0, 15).astype(np.uint8)
    q = np.where((d32 == 0)[..., None], np.uint8(8), q)
    out = np.empty((rows, cols // QK, 18), np.uint8)
    out[..., 0:2] = _f16_bytes(d32)
    out[..., 2:] = q[..., :16] | (q[..., 16:] << 4)
    return out.reshape(rows, -1)


def quantize_q2_dm(w: np.ndarray) -> np.ndarray:
    """2-bit scale/min blocks: d = (max-min)/3, m = min, q = round((w-m)/d) in 0..3.

    Byte j of the 8 payload bytes holds element j + 8p in bits [2p, 2p+2)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % QK == 0
    b = w.reshape(rows, cols // QK, QK)
    lo = b.min(axis=2)
    hi = b.max(axis=2)
    d32 = ((hi - lo) / np.float32(3.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(d32 > 0, np.float32(1.0) / d32, np.float32(0.0)).astype(np.float32)
    q = np.clip(_round_half_away((b - lo[..., None]) * inv[..., None]), 0, 3).astype(np.uint8)
    out = np.empty((rows, cols // QK, 12), np.uint8)
    out[..., 0:2] = _f16_bytes(d32)
    out[..., 2:4] = _f16_bytes(lo)
    qq = q.reshape(rows, cols // QK, 4, 8)  # [.., p, j] = element j + 8p
    out[..., 4:] = qq[..., 0, :] | (qq[..., 1, :] << 2) | (qq[..., 2, :] << 4) | (qq[..., 3, :] << 6)
    return out.reshape(rows, -1)


QUANTIZERS = {Q8_0: quantize_q8_0, Q4_0: quantize_q4_0, Q2_DM: quantize_q2_dm}


def quantize(qtype: int, w: np.ndarray) -> np.ndarray:
    return QUANTIZERS[qtype](w)


# ---------------------------------------------------------------------------
# workload definitions
# ---------------------------------------------------------------------------
@dataclass
class LinearCfg:
    name: str
    T: int
    K: int  # in-features
    N: int  # out-features
    qtype: int
    rank: int
    alpha: float
    seed: int = 0

    @property
    def scale(self) -> float:
        return self.alpha / self.rank


@dataclass
class MoECfg:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    qtype: int
    rank: int
    alpha: float
    zipf: float = 0.0  # exponent of the per-expert routing bias (0 = none)
    seed: int = 0

    @property
    def scale(self) -> float:
        return self.alpha / self.rank


@dataclass
class HeadCfg:
    name: str
    T: int
    H: int
    V: int
    qtype: int
    rank: int
    alpha: float
    chunk: int = 4096
    ignore_frac: float = 0.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return self.alpha / self.rank


# The five benchmark workloads.
LINEAR_Q8_0_T128 = LinearCfg("linear_q8_0_t128_1024x1024_r4", T=128, K=1024, N=1024, qtype=Q8_0, rank=4, alpha=8)
LINEAR_Q4_0_T2048 = LinearCfg("linear_q4_0_t2048_2048x6144_r4", T=2048, K=2048, N=6144, qtype=Q4_0, rank=4, alpha=8)
MOE_Q4_0_T2048 = MoECfg("moe_q4_0_t2048_h2048_e128k8_i768_r4", T=2048, H=2048, I=768, E=128, k=8,
                        qtype=Q4_0, rank=4, alpha=8)
MOE_Q2DM_T4096_ZIPF = MoECfg("moe_q2dm_t4096_h4096_e256k8_i1024_r8_zipf", T=4096, H=4096, I=1024, E=256,
                             k=8, qtype=Q2_DM, rank=8, alpha=16, zipf=1.0)
LMHEAD_Q8_0_T2048 = HeadCfg("lmhead_q8_0_t2048_h2048_v151936_r4", T=2048, H=2048, V=151936, qtype=Q8_0,
                            rank=4, alpha=8, chunk=4096)
CONFIGS = {c.name: c for c in (LINEAR_Q8_0_T128, LINEAR_Q4_0_T2048, MOE_Q4_0_T2048, MOE_Q2DM_T4096_ZIPF,
                               LMHEAD_Q8_0_T2048)}


def _normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def adapter_sigmas(n_in: int, large: bool) -> tuple[float, float]:
    """(sigma_A, sigma_B).  Default: A ~ N(0, sd 1/in), B ~ N(0, sd 0.01).
    The large-adapter variant reads the second argument of N(.,.) as a variance
    (A sd 1/sqrt(in), B sd 0.1) so the adapter term is a visible share of y."""
    if large:
        return 1.0 / math.sqrt(n_in), 0.1
    return 1.0 / n_in, 0.01


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------
def make_linear(cfg: LinearCfg, large_adapter: bool = False, w_sigma: float = 0.02) -> dict:
    """Draw order: x, W, A, B, dY (one PCG64 stream seeded with cfg.seed)."""
    rng = np.random.default_rng(cfg.seed)
    x = f32_to_bf16_bits(_normal(rng, (cfg.T, cfg.K), 1.0))
    w = _normal(rng, (cfg.N, cfg.K), w_sigma)
    blocks = quantize(cfg.qtype, w)
    del w
    sa, sb = adapter_sigmas(cfg.K, large_adapter)
    A = _normal(rng, (cfg.rank, cfg.K), sa)
    B = _normal(rng, (cfg.N, cfg.rank), sb)
    dy = f32_to_bf16_bits(_normal(rng, (cfg.T, cfg.N), 1.0))
    return dict(x=x, blocks=blocks, A=A, B=B, dy=dy, qtype=cfg.qtype, T=cfg.T, K=cfg.K, N=cfg.N,
                rank=cfg.rank, scale=np.float32(cfg.scale))


def _expert_weights(seed: int, e: int, cfg: MoECfg, large_adapter: bool, w_sigma: float):
    """Per-expert stream seeded with (seed, 1, e) so experts can be drawn in
    parallel.  Draw order: Wg, Wu, Wd, A_g, A_u, B_g, B_u, A_d, B_d."""
    rng = np.random.default_rng([seed, 1, e])
    H, I, r = cfg.H, cfg.I, cfg.rank
    wg = quantize(cfg.qtype, _normal(rng, (I, H), w_sigma))
    wu = quantize(cfg.qtype, _normal(rng, (I, H), w_sigma))
    wd = quantize(cfg.qtype, _normal(rng, (H, I), w_sigma))
    sah, sb = adapter_sigmas(H, large_adapter)
    sai, _ = adapter_sigmas(I, large_adapter)
    ag = _normal(rng, (r, H), sah)
    au = _normal(rng, (r, H), sah)
    bg = _normal(rng, (I, r), sb)
    bu = _normal(rng, (I, r), sb)
    ad = _normal(rng, (r, I), sai)
    bd = _normal(rng, (H, r), sb)
    return wg, wu, wd, ag, au, bg, bu, ad, bd


def zipf_bias(E: int, zeta: float, rng: np.random.Generator) -> np.ndarray:
    """Per-expert logit bias -zeta*ln(rank_e) with rank a seeded permutation of 1..E."""
    ranks = rng.permutation(E).astype(np.float64) + 1.0
    return (-zeta * np.log(ranks)).astype(np.float32)


def make_moe(cfg: MoECfg, large_adapter: bool = False, w_sigma: float = 0.02,
             threads: int | None = None, experts: list[int] | None = None) -> dict:
    """Token-side draws (stream seeded with (seed, 0)): logits, [zipf perm], x, dY.
    Expert-side draws: one stream per expert (see _expert_weights).
    `experts` restricts generation to a subset (others are left zero); used by
    sampled oracle checks that only need a few experts' weights."""
    rng = np.random.default_rng([cfg.seed, 0])
    T, H, I, E, r = cfg.T, cfg.H, cfg.I, cfg.E, cfg.rank
    logits = _normal(rng, (T, E), 1.0)
    bias = None
    if cfg.zipf:
        bias = zipf_bias(E, cfg.zipf, rng)
        logits = (logits + bias[None, :]).astype(np.float32)
    x = f32_to_bf16_bits(_normal(rng, (T, H), 1.0))
    dy = f32_to_bf16_bits(_normal(rng, (T, H), 1.0))
    bs = BLOCK_BYTES[cfg.qtype]
    wg = np.zeros((E, I, H // QK * bs), np.uint8)
    wu = np.zeros((E, I, H // QK * bs), np.uint8)
    wd = np.zeros((E, H, I // QK * bs), np.uint8)
    ag = np.zeros((E, r, H), np.float32)
    au = np.zeros((E, r, H), np.float32)
    bg = np.zeros((E, I, r), np.float32)
    bu = np.zeros((E, I, r), np.float32)
    ad = np.zeros((E, r, I), np.float32)
    bd = np.zeros((E, H, r), np.float32)
    todo = list(range(E)) if experts is None else sorted(set(int(e) for e in experts))

    def one(e):
        vals = _expert_weights(cfg.seed, e, cfg, large_adapter, w_sigma)
        for dst, v in zip((wg, wu, wd, ag, au, bg, bu, ad, bd), vals):
            dst[e] = v

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads > 1 and len(todo) > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, todo))
    else:
        for e in todo:
            one(e)
    return dict(logits=logits, bias=bias, x=x, dy=dy, wg=wg, wu=wu, wd=wd, ag=ag, au=au, bg=bg,
                bu=bu, ad=ad, bd=bd, qtype=cfg.qtype, T=T, H=H, I=I, E=E, k=cfg.k, rank=r,
                scale=np.float32(cfg.scale))


def make_head(cfg: HeadCfg, large_adapter: bool = False, w_sigma: float = 0.02,
              threads: int | None = None) -> dict:
    """Token stream (seed, 0): h, labels[, ignore mask].  Weight stream per
    4096-row chunk c: (seed, 2, c).  Adapter stream (seed, 3): A, B."""
    rng = np.random.default_rng([cfg.seed, 0])
    T, H, V, r = cfg.T, cfg.H, cfg.V, cfg.rank
    h = f32_to_bf16_bits(_normal(rng, (T, H), 1.0))
    labels = rng.integers(0, V, T).astype(np.int64)
    if cfg.ignore_frac > 0:
        ign = rng.random(T) < cfg.ignore_frac
        labels[ign] = -100
    bs = BLOCK_BYTES[cfg.qtype]
    blocks = np.empty((V, H // QK * bs), np.uint8)
    CH = 4096
    nch = (V + CH - 1) // CH

    def one(c):
        lo, hi = c * CH, min(V, (c + 1) * CH)
        crng = np.random.default_rng([cfg.seed, 2, c])
        blocks[lo:hi] = quantize(cfg.qtype, _normal(crng, (hi - lo, H), w_sigma))

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads > 1 and nch > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(nch)))
    else:
        for c in range(nch):
            one(c)
    arng = np.random.default_rng([cfg.seed, 3])
    sa, sb = adapter_sigmas(H, large_adapter)
    A = _normal(arng, (r, H), sa)
    B = _normal(arng, (V, r), sb)
    return dict(h=h, labels=labels, blocks=blocks, A=A, B=B, qtype=cfg.qtype, T=T, H=H, V=V,
                rank=r, scale=np.float32(cfg.scale), chunk=cfg.chunk)
