"""Build libgq.so (HIP, gfx950) in-tree.

    python -m quantized_base_lora_amd.build            # full rebuild
    python -m quantized_base_lora_amd.build --incremental
    python -m quantized_base_lora_amd.build --sanitize    # libgq_san.so

Every .hip under csrc/ is compiled by hipcc for gfx950 into _build/ (in
parallel), then linked into quantized_base_lora_amd/libgq.so.

--sanitize builds a checking variant, libgq_san.so: the C-ABI layer
(gq_api.hip: argument checks, workspace carving, error text) has its HOST
code compiled with AddressSanitizer and UndefinedBehaviorSanitizer, the
device code and the other objects are the regular ones.  The sanitizer
runtime is not linked in: load the library into a process started with
LD_PRELOAD=<clang's libclang_rt.asan .so> (see asan_runtime()).  It is a
host-side test build only; GPU code is never built with a sanitizer.
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
LIB_SAN = os.path.join(HERE, "libgq_san.so")
BUILD_SAN = os.path.join(HERE, "_build_san")
SAN_SOURCES = ("gq_api.hip",)
# host-only instrumentation: every sanitizer flag sits behind -Xarch_host
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]
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


def _compile(src: str, incremental: bool, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(p) for p in [src] + _headers())
        if os.path.getmtime(obj) >= newest:
            return obj
    cmd = [_hipcc(), *CFLAGS, *extra, "-c", src, "-o", obj]
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


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime of the ROCm clang (for LD_PRELOAD)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if c and os.path.exists(c):
            r = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("clang's AddressSanitizer runtime not found")


def build_sanitized(jobs: int | None = None, verbose: bool = False) -> str:
    """libgq_san.so: the regular objects (built incrementally) with the C-ABI
    layer's host code recompiled under ASan + UBSan."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(BUILD_SAN, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(16, max(1, os.cpu_count() or 1), len(srcs))

    def one(s):
        if os.path.basename(s) in SAN_SOURCES:
            return _compile(s, True, BUILD_SAN, SAN_FLAGS)
        return _compile(s, True)

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(one, srcs))
    tmp = LIB_SAN + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_SAN)
    if verbose:
        print(f"built {LIB_SAN} (host ASan/UBSan in {', '.join(SAN_SOURCES)})")
    return LIB_SAN


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("--sanitize", action="store_true", help="build libgq_san.so (host ASan/UBSan)")
    ap.add_argument("-j", "--jobs", type=int, default=None)
    a = ap.parse_args()
    if a.sanitize:
        build_sanitized(jobs=a.jobs, verbose=True)
    else:
        build(incremental=a.incremental, jobs=a.jobs, verbose=True)
    sys.exit(0)
