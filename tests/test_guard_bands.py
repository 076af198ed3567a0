"""The guard-band allocator that surrounds the binding's outputs and
workspaces in the GPU tests: it must return usable views and must notice a
write just outside a buffer.  The CPU case exercises the same logic on host
tensors; the GPU case writes into a margin with torch (a plain in-bounds
write into the larger allocation, never a kernel fault)."""
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import GuardedTorch  # noqa: E402


def _whole(t, nbytes):
    """uint8 view over the whole underlying allocation of t."""
    full = torch.empty(0, dtype=torch.uint8, device=t.device)
    full.set_(t.untyped_storage(), 0, (nbytes,))
    return full


def _exercise(device):
    g = GuardedTorch(torch, device_types=(device,))
    a = g.empty((3, 5), dtype=torch.float32, device=device)
    b = g.zeros(7, dtype=torch.bfloat16, device=device)
    c = g.empty((), dtype=torch.float32, device=device)
    assert a.shape == (3, 5) and b.shape == (7,) and c.shape == ()
    align = 256 if device == "cuda" else 64  # the allocators' own alignment is kept
    assert a.data_ptr() % align == 0 and b.data_ptr() % align == 0
    assert torch.all(b == 0)
    a.fill_(1.0)
    b.fill_(2.0)
    c.fill_(3.0)
    g.check()  # writes inside the buffers only: passes
    assert g.checked == 3
    d = g.empty(16, dtype=torch.int32, device=device)
    whole = _whole(d, 64 + 2 * GuardedTorch.GUARD)
    whole[GuardedTorch.GUARD + 64] = 0  # first byte after the buffer
    with pytest.raises(AssertionError, match="0 bytes changed before it, 1 after it"):
        g.check()
    e = g.empty(16, dtype=torch.int32, device=device)
    whole = _whole(e, 64 + 2 * GuardedTorch.GUARD)
    whole[GuardedTorch.GUARD - 1] = 0  # last byte before the buffer
    with pytest.raises(AssertionError, match="1 bytes changed before it, 0 after it"):
        g.check()


def test_guard_bands_on_host_tensors():
    _exercise("cpu")


@pytest.mark.gpu
def test_guard_bands_on_device_tensors():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _exercise("cuda")
