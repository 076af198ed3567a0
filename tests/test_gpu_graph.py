"""The entry points under HIP graph capture: each step (dense linear fwd+bwd,
routed MoE layer fwd+bwd, chunked LM head) is captured once and replayed
several times, with eager work of the program and host synchronisations
between the replays; every replay must reproduce the eager outputs bit for
bit (all reductions run in a fixed order, so the step is deterministic).
Nothing in the library clears memory with a memset node."""
import sys

import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_base_lora_amd as gq  # noqa: E402
from gpu_helpers import bf16_dev, f32_dev, i64_dev, u8_dev  # noqa: E402

REPLAYS = 3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _flat(out):
    """tensors of a step's (nested) outputs by name"""
    res = {}
    items = out.items() if isinstance(out, dict) else enumerate(out)
    for k, v in items:
        if isinstance(v, torch.Tensor):
            res[str(k)] = v
        elif isinstance(v, (dict, tuple, list)):
            for k2, t in _flat(v).items():
                res[f"{k}.{k2}"] = t
    return res


def _check_replays(step, noise):
    eager = {k: v.clone() for k, v in _flat(step()).items() if v is not None}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    captured = {k: v for k, v in _flat(out).items() if v is not None}
    assert captured.keys() == eager.keys()
    for rep in range(REPLAYS):
        noise()  # the program's own eager work between replays
        torch.cuda.synchronize()
        for v in captured.values():
            v.fill_(float("nan") if v.is_floating_point() else -7)
        g.replay()
        torch.cuda.synchronize()
        for k, v in captured.items():
            assert torch.equal(v, eager[k]), (rep, k)
        say(f"  replay {rep}: {len(captured)} outputs identical to eager")


def _noise():
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()


def test_graph_linear():
    cfg = synth.LinearCfg("g", T=300, K=512, N=520, qtype=1, rank=4, alpha=8)
    say("graph linear", cfg)
    inp = synth.make_linear(cfg)
    p = gq.Proj(cfg.qtype, cfg.N, cfg.K, u8_dev(inp["blocks"]), f32_dev(inp["A"]),
                f32_dev(inp["B"]), float(inp["scale"]))
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])

    def step():
        y, xa = gq.linear_lora_fwd(p, x)
        return (y, xa) + tuple(gq.linear_lora_bwd(p, x, xa, dy))

    _check_replays(step, _noise)


def test_graph_moe():
    cfg = synth.MoECfg("g", T=96, H=256, I=128, E=8, k=2, qtype=2, rank=4, alpha=8, zipf=1.1)
    say("graph moe", cfg)
    inp = synth.make_moe(cfg)
    s = float(inp["scale"])
    mk = lambda w, a, b, no, ni: gq.Proj(cfg.qtype, no, ni, u8_dev(w), f32_dev(a), f32_dev(b), s,
                                         cfg.E)
    wts = gq.MoEWeights(mk(inp["wg"], inp["ag"], inp["bg"], cfg.I, cfg.H),
                        mk(inp["wu"], inp["au"], inp["bu"], cfg.I, cfg.H),
                        mk(inp["wd"], inp["ad"], inp["bd"], cfg.H, cfg.I))
    x, dy, lg = bf16_dev(inp["x"]), bf16_dev(inp["dy"]), f32_dev(inp["logits"])

    def step():
        y, saved = gq.moe_ffn_fwd(wts, x, lg, cfg.k)
        return y, gq.moe_ffn_bwd(wts, x, dy, saved, cfg.k, cfg.E)

    _check_replays(step, _noise)


def test_graph_lmhead():
    cfg = synth.HeadCfg("g", T=200, H=128, V=1000, qtype=0, rank=4, alpha=8, chunk=384,
                        ignore_frac=0.1)
    say("graph lmhead", cfg)
    inp = synth.make_head(cfg)
    head = gq.Proj(cfg.qtype, cfg.V, cfg.H, u8_dev(inp["blocks"]), f32_dev(inp["A"]),
                   f32_dev(inp["B"]), float(inp["scale"]))
    h, lab = bf16_dev(inp["h"]), i64_dev(inp["labels"])
    ws = [None]

    def step():
        out = gq.lmhead_chunked_ce(head, h, lab, chunk_rows=cfg.chunk, ws=ws[0])
        ws[0] = out["ws"]
        return {k: v for k, v in out.items() if k != "ws"}

    _check_replays(step, _noise)
