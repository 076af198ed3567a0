import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden_blocks(path=os.path.join(GOLDEN, "dequant_handbuilt.txt")):
    """Parse the hand-built block fixture into a list of dicts."""
    cases, cur = [], None
    for raw in open(path):
        line = raw.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = {"name": rest}
            cases.append(cur)
        elif key == "qtype":
            cur["qtype"] = {"q8_0": 0, "q4_0": 1, "q2_dm": 2}[rest]
        elif key == "bytes":
            cur["bytes"] = bytes.fromhex(rest)
        elif key == "expect":
            cur["expect"] = [float(v) for v in rest.split()]
    return cases


@pytest.fixture(scope="session")
def golden_blocks():
    return read_golden_blocks()


@pytest.fixture(autouse=True)
def output_guard_bands(request):
    """Every output and workspace the binding allocates in a GPU test sits
    between guard bands of a known byte pattern, checked after the test."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    try:
        import torch
    except ImportError:
        yield
        return
    if not torch.cuda.is_available():
        yield
        return
    import quantized_base_lora_amd as gq
    from gpu_helpers import GuardedTorch
    guarded = GuardedTorch(torch)
    mp = pytest.MonkeyPatch()
    mp.setattr(gq, "torch", guarded)
    try:
        yield
    finally:
        mp.undo()
    guarded.check()
