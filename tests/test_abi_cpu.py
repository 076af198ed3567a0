"""C-ABI checks that need no GPU: the library loads, exports every function
include/gq.h declares, and rejects bad arguments on the host before any HIP
call (fake device addresses are never dereferenced on these paths)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_base_lora_amd", "libgq.so")
HDR = os.path.join(ROOT, "include", "gq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libgq.so not built")


def declared():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gq_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def gq():
    import quantized_base_lora_amd as q
    return q


def test_exports_match_header(gq):
    names = declared()
    assert len(names) >= 19
    lib = C.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert set(gq.EXPORTS) == set(names)


def test_version_and_block_bytes(gq):
    lib = gq.lib()
    assert lib.gq_version() >= 100
    assert [lib.gq_block_bytes(q) for q in (0, 1, 2)] == [34, 18, 12]
    assert lib.gq_block_bytes(7) == -1


FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced here


def proj(gq, **kw):
    d = dict(qtype=0, rank=4, n_out=64, n_in=128, w_blocks=FAKE, A=FAKE, B=FAKE, scale=2.0,
             n_experts=1)
    d.update(kw)
    return gq.LoraLinear(d["qtype"], d["rank"], d["n_out"], d["n_in"], d["w_blocks"], d["A"],
                         d["B"], d["scale"], d["n_experts"])


def test_dequant_validation(gq):
    lib = gq.lib()
    assert lib.gq_dequant(9, FAKE, 4, 64, 0, FAKE, None) == gq.GQ_EINVAL
    assert "qtype" in gq.last_error()
    assert lib.gq_dequant(0, FAKE, 4, 48, 0, FAKE, None) == gq.GQ_EINVAL
    assert lib.gq_dequant(0, FAKE, 4, 64, 5, FAKE, None) == gq.GQ_EINVAL
    assert lib.gq_dequant(0, None, 4, 64, 0, FAKE, None) == gq.GQ_EINVAL
    assert lib.gq_dequant(0, FAKE, 4, 64, 0, FAKE + 8, None) == gq.GQ_EINVAL
    assert lib.gq_dequant(0, FAKE, 0, 64, 0, FAKE, None) == gq.GQ_OK  # empty: no-op


def test_linear_validation(gq):
    lib = gq.lib()
    f = lib.gq_linear_lora_fwd
    L = proj(gq, rank=17)
    assert f(C.byref(L), FAKE, 8, FAKE, FAKE, None, 0, None) == gq.GQ_EINVAL
    assert "rank" in gq.last_error()
    L = proj(gq, n_in=96)
    assert f(C.byref(L), FAKE, 8, FAKE, FAKE, None, 0, None) == gq.GQ_ENOTSUP
    L = proj(gq, n_out=60)
    assert f(C.byref(L), FAKE, 8, FAKE, FAKE, None, 0, None) == gq.GQ_ENOTSUP
    L = proj(gq, qtype=5)
    assert f(C.byref(L), FAKE, 8, FAKE, FAKE, None, 0, None) == gq.GQ_EINVAL
    L = proj(gq, n_experts=2)
    assert f(C.byref(L), FAKE, 8, FAKE, FAKE, None, 0, None) == gq.GQ_EINVAL
    L = proj(gq, A=0)
    assert f(C.byref(L), FAKE, 8, FAKE, FAKE, None, 0, None) == gq.GQ_EINVAL
    L = proj(gq)
    assert f(C.byref(L), FAKE + 2, 8, FAKE, FAKE, None, 0, None) == gq.GQ_EINVAL  # misaligned x
    assert f(C.byref(L), None, 0, None, None, None, 0, None) == gq.GQ_OK  # T = 0
    b = lib.gq_linear_lora_bwd
    need = lib.gq_linear_lora_bwd_workspace_size(C.byref(L), 8)
    assert need > 0
    assert b(C.byref(L), FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, None, 0, None) == gq.GQ_EWORKSPACE
    assert b(C.byref(L), FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, FAKE, need - 1,
             None) == gq.GQ_EWORKSPACE
    assert "too small" in gq.last_error()
    assert b(C.byref(L), FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, FAKE + 16, need,
             None) == gq.GQ_EINVAL  # unaligned workspace


def test_route_validation(gq):
    lib = gq.lib()
    r = lib.gq_moe_route
    assert r(FAKE, 16, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == gq.GQ_EINVAL
    assert r(FAKE, 16, 2000, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == gq.GQ_EINVAL
    assert r(FAKE, 16, 8, 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == gq.GQ_EINVAL
    assert r(FAKE, 16, 64, 17, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == gq.GQ_EINVAL
    assert r(FAKE, 16, 8, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == gq.GQ_EWORKSPACE
    assert lib.gq_moe_route_workspace_size(4096, 256, 8) >= 128 * 256 * 4


def test_grouped_validation(gq):
    lib = gq.lib()
    P = (gq.LoraLinear * 2)(proj(gq, n_experts=4), proj(gq, n_experts=4, n_out=128))
    a = gq.GroupedFwdArgs(FAKE, FAKE, 2, FAKE, 64, FAKE, FAKE, FAKE, FAKE)
    assert lib.gq_grouped_mmq_lora_fwd(P, 2, 1, C.byref(a), FAKE, 1 << 20, None) == gq.GQ_EINVAL
    assert "differ" in gq.last_error()
    assert lib.gq_grouped_mmq_lora_fwd(P, 2, 0, C.byref(a), FAKE, 1 << 20, None) == gq.GQ_EINVAL
    P1 = (gq.LoraLinear * 1)(proj(gq, n_experts=2000))
    assert lib.gq_grouped_mmq_lora_fwd(P1, 1, 0, C.byref(a), FAKE, 1 << 20, None) == gq.GQ_EINVAL
    b = gq.GroupedBwdArgs()
    b.offsets = FAKE
    b.M = 64
    b.gather_div = 1
    P3 = (gq.LoraLinear * 3)(proj(gq, n_experts=4, n_out=128, n_in=64),
                             proj(gq, n_experts=4, n_out=64, n_in=128),
                             proj(gq, n_experts=4, n_out=64, n_in=128))
    assert lib.gq_grouped_mmq_lora_bwd(P3, 3, 0, C.byref(b), None, 0, None) == gq.GQ_EWORKSPACE
    assert lib.gq_grouped_mmq_lora_bwd(P3, 2, 0, C.byref(b), None, 0, None) == gq.GQ_EINVAL
    assert lib.gq_grouped_mmq_lora_bwd(P3, 3, 7, C.byref(b), None, 0, None) == gq.GQ_EINVAL


def test_lmhead_validation(gq):
    lib = gq.lib()
    L = proj(gq, n_out=1024, n_in=128)
    ce = lib.gq_lmhead_chunked_ce
    assert ce(C.byref(L), FAKE, FAKE, 8, 0, -100, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
              None) == gq.GQ_EINVAL
    assert ce(C.byref(L), FAKE, FAKE, 8, 256, -100, 1.0, FAKE, FAKE, FAKE, None, FAKE, FAKE,
              1 << 30, None) == gq.GQ_EINVAL
    need = lib.gq_lmhead_chunked_ce_workspace_size(C.byref(L), 8, 256)
    assert ce(C.byref(L), FAKE, FAKE, 8, 256, -100, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
              need - 256, None) == gq.GQ_EWORKSPACE


def test_workspace_never_reaches_a_full_precision_weight(gq):
    """The fused kernels decode blocks into LDS/registers: no workspace query
    ever asks for as much memory as a bf16 copy of the weight (ai-manual.ru:
    the fused kernel never materialises the fp16 weights)."""
    lib = gq.lib()
    L = proj(gq, qtype=1, n_out=6144, n_in=2048)
    bf16_w = 6144 * 2048 * 2
    assert lib.gq_linear_lora_fwd_workspace_size(C.byref(L), 2048) < bf16_w
    assert lib.gq_linear_lora_bwd_workspace_size(C.byref(L), 2048) < bf16_w
    P3 = (gq.LoraLinear * 3)(proj(gq, qtype=1, n_experts=128, n_out=2048, n_in=768),
                             proj(gq, qtype=1, n_experts=128, n_out=768, n_in=2048),
                             proj(gq, qtype=1, n_experts=128, n_out=768, n_in=2048))
    experts_bf16 = 128 * 3 * 768 * 2048 * 2
    assert lib.gq_grouped_mmq_lora_bwd_workspace_size(P3, 3, 0, 16384) < experts_bf16
    assert lib.gq_grouped_mmq_lora_bwd_workspace_size(P3, 2, 1, 16384) < experts_bf16
    H = proj(gq, qtype=0, n_out=151936, n_in=2048)
    assert lib.gq_lmhead_chunked_ce_workspace_size(C.byref(H), 2048, 4096) < 151936 * 2048 * 2


def test_rmsnorm_validation(gq):
    lib = gq.lib()
    assert lib.gq_rmsnorm_fwd(FAKE, FAKE, 4, 12, 1e-6, FAKE, FAKE, None) == gq.GQ_EINVAL
    assert "multiple of 8" in gq.last_error()
    assert lib.gq_rmsnorm_fwd(FAKE, FAKE, 4, 64, -1.0, FAKE, FAKE, None) == gq.GQ_EINVAL
    assert lib.gq_rmsnorm_fwd(FAKE + 2, FAKE, 4, 64, 1e-6, FAKE, FAKE, None) == gq.GQ_EINVAL
    assert "aligned" in gq.last_error()
    assert lib.gq_rmsnorm_fwd(None, FAKE, 4, 64, 1e-6, FAKE, FAKE, None) == gq.GQ_EINVAL
    assert lib.gq_rmsnorm_fwd(FAKE, FAKE, 0, 64, 1e-6, FAKE, FAKE, None) == gq.GQ_OK  # T = 0: no-op
    assert lib.gq_rmsnorm_bwd(FAKE, FAKE, FAKE, FAKE, -1, 64, FAKE, None) == gq.GQ_EINVAL
    assert lib.gq_rmsnorm_bwd(FAKE, FAKE, FAKE, None, 4, 64, FAKE, None) == gq.GQ_EINVAL


def test_adamw8bit_validation(gq):
    lib = gq.lib()
    st = lib.gq_adamw8bit_step
    args = [FAKE] * 6
    assert st(*args, 100, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == gq.GQ_EINVAL  # step 0
    assert "step" in gq.last_error()
    assert st(*args, 100, 1, 1e-3, 1.0, 0.999, 1e-8, 0.0, None) == gq.GQ_EINVAL  # beta1 = 1
    assert st(*args, 100, 1, 1e-3, 0.9, 0.999, 0.0, 0.0, None) == gq.GQ_EINVAL   # eps = 0
    assert st(*args, -1, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == gq.GQ_EINVAL
    assert st(None, *args[1:], 100, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == gq.GQ_EINVAL
    assert st(*args, 0, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == gq.GQ_OK  # n = 0: no-op


def test_noalloc_rejects_oversized_shapes_on_the_host(gq):
    lib = gq.lib()
    cap = lib.gq_noalloc_scratch_bytes()
    L = proj(gq, qtype=1, rank=16, n_out=1 << 20, n_in=1 << 16)
    T = 1 << 20
    assert lib.gq_linear_lora_bwd_workspace_size(C.byref(L), T) > cap
    rc = lib.gq_linear_lora_bwd_noalloc(C.byref(L), FAKE, FAKE, FAKE, T, FAKE, FAKE, FAKE, None)
    assert rc == gq.GQ_EWORKSPACE and "scratch" in gq.last_error()
    assert lib.gq_linear_lora_bwd_noalloc(C.byref(proj(gq, rank=17)), FAKE, FAKE, FAKE, 8, FAKE, FAKE,
                                          FAKE, None) == gq.GQ_EINVAL
