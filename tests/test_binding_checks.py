"""The Python binding checks every tensor before its pointer reaches the
library (CPU: no GPU needed, nothing is launched): dtype, exact shape,
contiguity and the byte size of the weight blocks, then that it is a GPU
tensor."""
import pytest

torch = pytest.importorskip("torch")
import quantized_base_lora_amd as gq  # noqa: E402


def test_expect_reports_each_mismatch():
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="dtype"):
        gq._expect(x.float(), "x", torch.bfloat16, (None, 64))
    with pytest.raises(ValueError, match="shape"):
        gq._expect(x, "x", torch.bfloat16, (None, 128))
    with pytest.raises(ValueError, match="shape"):
        gq._expect(x, "x", torch.bfloat16, (5, 64))
    with pytest.raises(ValueError, match="rows"):
        gq._expect(x, "x", torch.bfloat16, (None, 64), min_rows=8)
    with pytest.raises(ValueError, match="contiguous"):
        gq._expect(torch.zeros((64, 4), dtype=torch.bfloat16).t(), "x", torch.bfloat16, (4, 64))
    with pytest.raises(ValueError, match="GPU"):
        gq._expect(x, "x", torch.bfloat16, (4, 64))
    with pytest.raises(TypeError, match="Tensor"):
        gq._expect(x.numpy() if False else [1, 2], "x", torch.bfloat16)


def proj(n_out=64, n_in=128, qtype=gq.Q4_0, r=4, E=1, nbytes=None):
    bs = gq.BLOCK_BYTES[qtype]
    nb = E * n_out * (n_in // 32) * bs if nbytes is None else nbytes
    lead = (E,) if E > 1 else ()
    return gq.Proj(qtype, n_out, n_in, torch.zeros(nb, dtype=torch.uint8),
                   torch.zeros(lead + (r, n_in)), torch.zeros(lead + (n_out, r)), 2.0, E)


def test_proj_check():
    with pytest.raises(ValueError, match="blocks"):
        proj(nbytes=100).check()
    with pytest.raises(ValueError, match="rank"):
        proj(r=17).check()
    p = proj()
    p.A = torch.zeros((4, 64))
    with pytest.raises(ValueError, match="A"):
        p.check()
    p = proj(E=4)
    p.B = torch.zeros((3, 64, 4))
    with pytest.raises(ValueError, match="B"):
        p.check()
    p = proj()
    p.A = p.A.double()
    with pytest.raises(TypeError, match="A"):
        p.check()
    with pytest.raises(ValueError, match="GPU"):  # everything right but the device
        proj().check()


def test_entry_points_refuse_host_tensors_before_the_library():
    p = proj()
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    for call in (lambda: gq.linear_lora_fwd(p, x),
                 lambda: gq.linear_lora_bwd(p, x, torch.zeros((4, 4)), torch.zeros((4, 64), dtype=torch.bfloat16)),
                 lambda: gq.moe_route(torch.zeros((4, 8)), 2),
                 lambda: gq.rmsnorm_fwd(x, torch.ones(128)),
                 lambda: gq.dequant(gq.Q4_0, torch.zeros(18 * 4, dtype=torch.uint8), 1, 128)):
        with pytest.raises(ValueError, match="GPU"):
            call()
    with pytest.raises(TypeError, match="dtype"):
        gq.moe_route(torch.zeros((4, 8), dtype=torch.float64), 2)
    with pytest.raises(ValueError, match="bytes"):
        gq.dequant(gq.Q4_0, torch.zeros(10, dtype=torch.uint8), 1, 128)
