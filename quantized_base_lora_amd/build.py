"""Build libgq.so (HIP, gfx950) in-tree.

    python -m quantized_base_lora_amd.build            # full rebuild
    python -m quantized_base_lora_amd.build --incremental

Every .hip under csrc/ is compiled by hipcc for gfx950 into _build/ (in
parallel), then linked into quantized_base_lora_amd/libgq.so.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgq.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = os.environ.get("GQ_OFFLOAD_ARCH", "gfx950")
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"-I{INCLUDE}",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libgq)")


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _headers():
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    hs.append(os.path.join(INCLUDE, "gq.h"))
    return hs


def _compile(src: str, incremental: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(p) for p in [src] + _headers())
        if os.path.getmtime(obj) >= newest:
            return obj
    cmd = [_hipcc(), *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "not a recognized feature" not in l)
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{msg}")
    return obj


def build(incremental: bool = False, jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(16, max(1, os.cpu_count() or 1), len(srcs))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(objs)} objects")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    a = ap.parse_args()
    build(incremental=a.incremental, jobs=a.jobs, verbose=True)
    sys.exit(0)
