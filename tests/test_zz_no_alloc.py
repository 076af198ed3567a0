"""The no-allocation variant of the fast LoRA backward
(gq_linear_lora_bwd_noalloc, scratch in the library's fixed device array)
against the workspace entry point gq_linear_lora_bwd on the same inputs:
outputs bitwise equal, on two calls in a row (the second smaller, so it
runs on scratch the first one left behind), plus the oracle's bar on the
smaller case."""
import sys

import numpy as np
import pytest

import synth
from oracle import linear as ol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import quantized_base_lora_amd as gq  # noqa: E402
from gpu_helpers import bf16_dev, check, f32_dev, host, u8_dev  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(cfg, large):
    inp = synth.make_linear(cfg, large_adapter=large)
    p = gq.Proj(inp["qtype"], inp["N"], inp["K"], u8_dev(inp["blocks"]), f32_dev(inp["A"]),
                f32_dev(inp["B"]), float(inp["scale"]))
    x, dy = bf16_dev(inp["x"]), bf16_dev(inp["dy"])
    y, xa = gq.linear_lora_fwd(p, x)
    ref = gq.linear_lora_bwd(p, x, xa, dy)
    # outputs preallocated, so the no-allocation call allocates nothing
    out = (torch.full((cfg.T, cfg.K), float("nan"), dtype=torch.bfloat16, device=x.device),
           torch.full((cfg.rank, cfg.K), float("nan"), dtype=torch.float32, device=x.device),
           torch.full((cfg.N, cfg.rank), float("nan"), dtype=torch.float32, device=x.device))
    got = gq.linear_lora_bwd_noalloc(p, x, xa, dy, *out)
    torch.cuda.synchronize()
    for name, a, b in zip(("dx", "dA", "dB"), got, ref):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), name
    return inp, got


def test_noalloc_matches_workspace_entry_point_twice():
    big = synth.LinearCfg("noalloc_big", T=2048, K=2048, N=6144, qtype=synth.Q4_0, rank=4, alpha=8)
    small = synth.LinearCfg("noalloc_small", T=77, K=192, N=136, qtype=synth.Q8_0, rank=16, alpha=16)
    say("noalloc", big.name)
    _run(big, False)
    say("noalloc", small.name)
    inp, (dx, dA, dB) = _run(small, True)
    r = ol.run(inp)
    check("dx", host(dx), r["dx"])
    check("dA", host(dA), r["dA"])
    check("dB", host(dB), r["dB"])


def test_noalloc_rejects_shapes_beyond_the_scratch():
    lib = gq.lib()
    cap = lib.gq_noalloc_scratch_bytes()
    assert cap == 32 << 20
    dev = torch.zeros(16, device="cuda")
    L = gq.LoraLinear(1, 16, 1 << 20, 1 << 16, dev.data_ptr(), dev.data_ptr(), dev.data_ptr(), 1.0, 1)
    T = 1 << 20
    import ctypes as C
    assert lib.gq_linear_lora_bwd_workspace_size(C.byref(L), T) > cap
    rc = lib.gq_linear_lora_bwd_noalloc(C.byref(L), dev.data_ptr(), dev.data_ptr(), dev.data_ptr(), T,
                                        dev.data_ptr(), dev.data_ptr(), dev.data_ptr(), None)
    assert rc == gq.GQ_EWORKSPACE and "scratch" in gq.last_error()
