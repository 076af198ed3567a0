"""fp64 CPU oracle for LoRA over a frozen GGUF block-quantised base.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or execute this package; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

It is a plain, slow, obviously-correct restatement of what the method
computes, written from the pages (page 2, "Show HN: LoRA over GGUF - Train
Qwen3.8-Flash-Next in 40G VRAM", section "Things involved in the training":
quantised matrix products over the GGUF blocks after llama.cpp's MMQ, dense
and grouped by expert; Unsloth's fast LoRA backward for linear and MoE
layers; top-k MoE routing after OpenAI's triton-kernels; a chunked cross
entropy after Liger Kernel's that consumes the MMQ output; no
load-balancing loss).  Everything is computed in float64 from the exact bytes and
bf16 values the GPU receives.  It shares no code with the HIP path: the only
module both sides import is ``synth`` (seeded inputs, no method arithmetic).

Modules:
  blocks   - block decode (Q8_0, Q4_0, 2-bit scale/min)
  linear   - fused linear forward and the fast LoRA backward
  routing  - softmax top-k, stable expert sort, offsets, positions; backward
  moe      - grouped expert FFN forward/backward and a per-token brute force
  lmhead   - LM head with chunked online log-sum-exp cross entropy
  rmsnorm  - RMS normalisation with a frozen weight (the step before a linear)
  adamw8bit - AdamW with 8-bit block-wise quantised states (the adapters' optimizer)

Every function is pinned by tests under tests/ (marked "not gpu") to values
fixed independently of the oracle: hand-built blocks, closed forms, brute
force and finite differences.
"""
from . import blocks, linear, routing, moe, lmhead, rmsnorm, adamw8bit  # noqa: F401
