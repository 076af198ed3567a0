"""C-ABI checks that need no GPU: the library loads, exports every function
include/gq.h declares, and rejects bad arguments on the host before any HIP
call (fake device addresses are never dereferenced on these paths)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.environ.get("GQ_LIB") or os.path.join(ROOT, "quantized_base_lora_amd", "libgq.so")
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
    L = proj(gq, n_in=80)
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


def _bad(a):
    """An address aligned to a/2 but not to a."""
    return FAKE + a // 2


def test_each_pointer_alignment_is_checked_and_named(gq):
    """One misaligned argument at a time: GQ_EINVAL before any HIP call, with
    the argument's name in the message."""
    lib = gq.lib()
    L = proj(gq)
    big = 1 << 30

    def expect(call, argname):
        assert call() == gq.GQ_EINVAL, argname
        assert argname in gq.last_error() and "aligned" in gq.last_error(), gq.last_error()

    # dequant: blocks, out
    for i, (nm, a) in enumerate((("blocks", 2), ("out", 16))):
        args = [FAKE, FAKE]
        args[i] = _bad(a)
        expect(lambda: lib.gq_dequant(0, args[0], 4, 64, 0, args[1], None), nm)
    # linear forward: x, y, xa
    for i, (nm, a) in enumerate((("x", 16), ("y", 2), ("xa", 4))):
        args = [FAKE] * 3
        args[i] = _bad(a)
        expect(lambda: lib.gq_linear_lora_fwd(C.byref(L), args[0], 8, args[1], args[2], None, 0, None), nm)
    # linear backward: x, xa, dy, dx, dA, dB
    for i, (nm, a) in enumerate((("x", 16), ("xa", 4), ("dy", 16), ("dx", 2), ("dA", 4), ("dB", 4))):
        args = [FAKE] * 6
        args[i] = _bad(a)
        expect(lambda: lib.gq_linear_lora_bwd(C.byref(L), args[0], args[1], args[2], 8, args[3], args[4],
                                              args[5], FAKE, big, None), nm)
    # projection pointers
    for fld, a in (("w_blocks", 4), ("A", 16), ("B", 16)):
        Lb = proj(gq, **{fld: _bad(a)})
        expect(lambda: lib.gq_linear_lora_fwd(C.byref(Lb), FAKE, 8, FAKE, FAKE, None, 0, None), fld)
    # routing
    for i, nm in enumerate(("logits", "ids", "w", "sorted", "offsets", "pos")):
        args = [FAKE] * 6
        args[i] = _bad(4)
        expect(lambda: lib.gq_moe_route(args[0], 16, 8, 2, args[1], args[2], args[3], args[4], args[5], FAKE,
                                        big, None), nm)
    for i, nm in enumerate(("ids", "w", "dw", "dlogits")):
        args = [FAKE] * 4
        args[i] = _bad(4)
        expect(lambda: lib.gq_moe_route_bwd(args[0], args[1], args[2], 16, 8, 2, args[3], None), nm)
    # combines
    for i, (nm, a) in enumerate((("o", 16), ("w", 4), ("pos", 4), ("y", 16))):
        args = [FAKE] * 4
        args[i] = _bad(a)
        expect(lambda: lib.gq_moe_combine_fwd(args[0], args[1], args[2], 16, 2, 64, args[3], None), nm)
    for i, (nm, a) in enumerate((("dxrows", 16), ("pos", 4), ("dx", 16))):
        args = [FAKE] * 3
        args[i] = _bad(a)
        expect(lambda: lib.gq_moe_combine_bwd(args[0], args[1], 16, 2, 64, args[2], None), nm)
    # RMS normalisation
    for i, (nm, a) in enumerate((("x", 16), ("w", 16), ("y", 16), ("rstd", 4))):
        args = [FAKE] * 4
        args[i] = _bad(a)
        expect(lambda: lib.gq_rmsnorm_fwd(args[0], args[1], 4, 64, 1e-6, args[2], args[3], None), nm)
    for i, (nm, a) in enumerate((("dy", 16), ("x", 16), ("w", 16), ("rstd", 4), ("dx", 16))):
        args = [FAKE] * 5
        args[i] = _bad(a)
        expect(lambda: lib.gq_rmsnorm_bwd(args[0], args[1], args[2], args[3], 4, 64, args[4], None), nm)
    # AdamW
    for i, nm in ((0, "p"), (1, "g"), (4, "m_scale"), (5, "v_scale")):
        args = [FAKE] * 6
        args[i] = _bad(4)
        expect(lambda: lib.gq_adamw8bit_step(*args, 100, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None), nm)
    # LM head
    for i, (nm, a) in enumerate((("h", 16), ("labels", 8), ("loss", 4), ("lse", 4), ("dh", 2), ("dA", 4),
                                 ("dB", 4))):
        args = [FAKE] * 7
        args[i] = _bad(a)
        expect(lambda: lib.gq_lmhead_chunked_ce(C.byref(proj(gq, n_out=1024)), args[0], args[1], 8, 256, -100,
                                                1.0, args[2], args[3], args[4], args[5], args[6], FAKE, big,
                                                None), nm)
    # grouped forward
    P2 = (gq.LoraLinear * 2)(proj(gq, n_experts=4), proj(gq, n_experts=4))
    fields = (("in", "inp", 16), ("out", "out", 2), ("save_g", "save_g", 2), ("save_u", "save_u", 2),
              ("xa", "xa", 4), ("gather", "gather", 4), ("offsets", "offsets", 4))
    for nm, fld, a in fields:
        ga = gq.GroupedFwdArgs(FAKE, FAKE, 2, FAKE, 64, FAKE, FAKE, FAKE, FAKE)
        setattr(ga, fld, _bad(a))
        expect(lambda: lib.gq_grouped_mmq_lora_fwd(P2, 2, 1, C.byref(ga), FAKE, big, None), nm)
    # grouped backward, both modes
    P3 = (gq.LoraLinear * 3)(proj(gq, n_experts=4, n_out=128, n_in=64),
                             proj(gq, n_experts=4, n_out=64, n_in=128),
                             proj(gq, n_experts=4, n_out=64, n_in=128))
    down = (("dy", 16), ("g", 16), ("u", 16), ("h", 16), ("dg", 16), ("du", 16), ("w_flat", 4), ("sorted", 4),
            ("xa_d", 4), ("dw_flat", 4), ("dA_d", 4), ("dB_d", 4), ("dgB", 4), ("duB", 4), ("gather", 4))
    gu = (("x", 16), ("dg", 16), ("du", 16), ("dxrows", 2), ("xa", 4), ("dgB", 4), ("duB", 4), ("dA_g", 4),
          ("dB_g", 4), ("dA_u", 4), ("dB_u", 4), ("gather", 4))
    for mode, projs, n, table in ((0, P3, 3, down), (1, (gq.LoraLinear * 2)(P3[1], P3[2]), 2, gu)):
        for nm, a in table:
            b = gq.GroupedBwdArgs()
            for f, _ in gq.GroupedBwdArgs._fields_:
                if f not in ("M", "gather_div"):
                    setattr(b, f, FAKE)
            b.M = 64
            b.gather_div = 1
            setattr(b, nm, _bad(a))
            expect(lambda: lib.gq_grouped_mmq_lora_bwd(projs, n, mode, C.byref(b), FAKE, big, None), nm)
