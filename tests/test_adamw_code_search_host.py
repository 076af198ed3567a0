"""Exhaustive host check of the 8-bit AdamW kernel's code search (CPU).

The kernel finds the nearest code with a table lookup and a linear estimate
instead of a bisection; tests/host/adamw_code_search.hip compiles that same
search for the host and compares it with a bisection of the same book on
every float in [0, 1 + 4 ulp], for both books.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_direct_code_search_matches_bisection(tmp_path):
    exe = tmp_path / "adamw_code_search"
    cmd = [HIPCC, "-O2", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "quantized_base_lora_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "adamw_code_search.hip"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert out.stdout.count(" 0 mismatches") == 2
