"""The C-ABI checks of test_abi_cpu.py, run again against libgq_san.so: the
same library with the host code of its C-ABI layer built under
AddressSanitizer and UndefinedBehaviorSanitizer.  Any out-of-bounds access,
use-after-free or undefined behaviour on those host paths (argument checks,
workspace sizing and carving, error text formatting) aborts the child
process and fails this test.  No GPU is used."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc needed to build the sanitized library")


def test_abi_checks_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    from quantized_base_lora_amd import build as b
    lib = b.build_sanitized()
    env = dict(os.environ)
    env.update(GQ_LIB=lib, LD_PRELOAD=b.asan_runtime(),
               # the interpreter's own allocations are not this library's leaks
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
