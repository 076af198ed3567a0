"""The library's environment switches.

GQ_TRACE=2 prints one line per entry point call; GQ_DEBUG=1 synchronises
after each call and returns the device error word as GQ_EDEVICE.  The
switches are read once per process, so each case runs in a child process.
The CPU case calls an entry point with a bad argument (no HIP call is made);
the GPU case drives the two device error words (inconsistent expert offsets,
a label outside the vocabulary) and a valid call."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_base_lora_amd", "libgq.so")


def run_child(code: str, **env):
    e = dict(os.environ)
    e.update(env)
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code)], cwd=ROOT, env=e,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgq.so not built")
def test_trace_lines_on_the_host():
    r = run_child("""
        import ctypes as C
        import quantized_base_lora_amd as gq
        lib = gq.lib()
        L = gq.LoraLinear(0, 17, 64, 128, 0x7F0000000000, 0x7F0000000000, 0x7F0000000000, 2.0, 1)
        rc = lib.gq_linear_lora_fwd(C.byref(L), 0x7F0000000000, 8, 0x7F0000000000, 0x7F0000000000,
                                    None, 0, None)
        print("rc", rc)
    """, GQ_TRACE="2")
    assert r.returncode == 0, r.stderr
    assert "rc -1" in r.stdout
    assert "[gq] gq_linear_lora_fwd -> -1: " in r.stderr and "rank" in r.stderr, r.stderr


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgq.so not built")
def test_switches_off_print_nothing():
    r = run_child("""
        import ctypes as C
        import quantized_base_lora_amd as gq
        L = gq.LoraLinear(0, 17, 64, 128, 0x7F0000000000, 0x7F0000000000, 0x7F0000000000, 2.0, 1)
        print("rc", gq.lib().gq_linear_lora_fwd(C.byref(L), 0x7F0000000000, 8, 0x7F0000000000,
                                                0x7F0000000000, None, 0, None))
    """, GQ_TRACE="0", GQ_DEBUG="0")
    assert r.returncode == 0 and "rc -1" in r.stdout
    assert "[gq]" not in r.stderr


@pytest.mark.gpu
def test_debug_switch_reports_device_errors_synchronously():
    r = run_child("""
        import sys
        import numpy as np
        import torch
        sys.path.insert(0, "tests")
        import synth
        import quantized_base_lora_amd as gq
        from gpu_helpers import bf16_dev, f32_dev, i32_dev, i64_dev, u8_dev
        print("case: grouped offsets", flush=True)
        cfg = synth.MoECfg("t", T=32, H=128, I=64, E=4, k=2, qtype=1, rank=4, alpha=8)
        inp = synth.make_moe(cfg)
        s, qt, E, H, I = float(inp["scale"]), cfg.qtype, cfg.E, cfg.H, cfg.I
        gate = gq.Proj(qt, I, H, u8_dev(inp["wg"]), f32_dev(inp["ag"]), f32_dev(inp["bg"]), s, E)
        up = gq.Proj(qt, I, H, u8_dev(inp["wu"]), f32_dev(inp["au"]), f32_dev(inp["bu"]), s, E)
        x = bf16_dev(inp["x"])
        M = cfg.T * cfg.k
        gather = torch.arange(M, dtype=torch.int32, device="cuda")
        try:
            gq.grouped_mmq_lora_fwd([gate, up], gq.EPI_SWIGLU, x, gather, cfg.k,
                                    i32_dev(np.array([0, 30, 20, 50, M])), M)
            print("bad offsets: no error")
        except gq.GQError as e:
            print("bad offsets:", e.code, str(e))
        gq.grouped_mmq_lora_fwd([gate, up], gq.EPI_SWIGLU, x, gather, cfg.k,
                                i32_dev(np.array([0, 10, 20, 30, M])), M)
        print("good offsets: ok")
        print("case: lm head label", flush=True)
        hc = synth.HeadCfg("t", T=16, H=64, V=256, qtype=0, rank=4, alpha=8, chunk=128)
        hi = synth.make_head(hc)
        hi["labels"][3] = 999
        head = gq.Proj(0, 256, 64, u8_dev(hi["blocks"]), f32_dev(hi["A"]), f32_dev(hi["B"]),
                       float(hi["scale"]))
        try:
            gq.lmhead_chunked_ce(head, bf16_dev(hi["h"]), i64_dev(hi["labels"]), chunk_rows=128)
            print("bad label: no error")
        except gq.GQError as e:
            print("bad label:", e.code, str(e))
        hi["labels"][3] = 5
        gq.lmhead_chunked_ce(head, bf16_dev(hi["h"]), i64_dev(hi["labels"]), chunk_rows=128)
        print("good labels: ok")
    """, GQ_DEBUG="1", GQ_TRACE="2")
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "bad offsets: -5 gq error -5: gq_grouped_mmq_lora_fwd (GQ_DEBUG): device error word" in r.stdout
    assert "good offsets: ok" in r.stdout
    assert "bad label: -5 gq error -5: gq_lmhead_chunked_ce (GQ_DEBUG): device error word" in r.stdout
    assert "good labels: ok" in r.stdout
    assert "[gq] gq_grouped_mmq_lora_fwd -> 0" in r.stderr
