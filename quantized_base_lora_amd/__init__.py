"""Python binding of libgq (LoRA over a frozen GGUF block-quantised base, MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libgq.so (C ABI declared in include/gq.h).  PyTorch provides device
memory and the current HIP stream.  The library must be built
(`python -m quantized_base_lora_amd.build`); importing the binding without it
raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GQ_LIB names another build of the same library (e.g. the host-sanitized
# libgq_san.so); the default is the in-tree libgq.so.
LIB_PATH = os.environ.get("GQ_LIB") or os.path.join(_HERE, "libgq.so")

GQ_OK, GQ_EINVAL, GQ_ENOTSUP, GQ_EWORKSPACE, GQ_EHIP, GQ_EDEVICE = 0, -1, -2, -3, -4, -5
Q8_0, Q4_0, Q2_DM = 0, 1, 2
F32, BF16 = 0, 1
EPI_NONE, EPI_SWIGLU = 0, 1
BWD_DOWN_SWIGLU, BWD_GATEUP = 0, 1
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q2_DM: 12}

EXPORTS = (
    "gq_version", "gq_last_error", "gq_block_bytes", "gq_profile_mmq_events", "gq_dequant",
    "gq_linear_lora_fwd_workspace_size", "gq_linear_lora_fwd",
    "gq_linear_lora_bwd_workspace_size", "gq_linear_lora_bwd",
    "gq_noalloc_scratch_bytes", "gq_linear_lora_bwd_noalloc",
    "gq_moe_route_workspace_size", "gq_moe_route", "gq_moe_route_bwd",
    "gq_moe_combine_fwd", "gq_moe_combine_bwd",
    "gq_grouped_mmq_lora_fwd_workspace_size", "gq_grouped_mmq_lora_fwd",
    "gq_grouped_mmq_lora_bwd_workspace_size", "gq_grouped_mmq_lora_bwd",
    "gq_lmhead_chunked_ce_workspace_size", "gq_lmhead_chunked_ce",
    "gq_rmsnorm_fwd", "gq_rmsnorm_bwd", "gq_adamw8bit_step",
)


class GQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gq error {code}: {msg}")
        self.code = code


class LoraLinear(C.Structure):
    _fields_ = [("qtype", C.c_int32), ("rank", C.c_int32), ("n_out", C.c_int64),
                ("n_in", C.c_int64), ("w_blocks", C.c_void_p), ("A", C.c_void_p),
                ("B", C.c_void_p), ("scale", C.c_float), ("n_experts", C.c_int32)]


class GroupedFwdArgs(C.Structure):
    _fields_ = [("inp", C.c_void_p), ("gather", C.c_void_p), ("gather_div", C.c_int32),
                ("offsets", C.c_void_p), ("M", C.c_int64), ("out", C.c_void_p),
                ("save_g", C.c_void_p), ("save_u", C.c_void_p), ("xa", C.c_void_p)]


class GroupedBwdArgs(C.Structure):
    _fields_ = [("offsets", C.c_void_p), ("M", C.c_int64), ("gather", C.c_void_p),
                ("gather_div", C.c_int32),
                ("dy", C.c_void_p), ("w_flat", C.c_void_p), ("sorted", C.c_void_p),
                ("g", C.c_void_p), ("u", C.c_void_p), ("h", C.c_void_p), ("xa_d", C.c_void_p),
                ("dw_flat", C.c_void_p), ("dA_d", C.c_void_p), ("dB_d", C.c_void_p),
                ("dg", C.c_void_p), ("du", C.c_void_p), ("dgB", C.c_void_p), ("duB", C.c_void_p),
                ("x", C.c_void_p), ("xa", C.c_void_p), ("dxrows", C.c_void_p),
                ("dA_g", C.c_void_p), ("dB_g", C.c_void_p), ("dA_u", C.c_void_p),
                ("dB_u", C.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgq.so and declare its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libgq.so not built at {path}; run python -m quantized_base_lora_amd.build")
    lib = C.CDLL(path)
    vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    P = C.POINTER
    sig = {
        "gq_version": (C.c_int, []),
        "gq_last_error": (C.c_char_p, []),
        "gq_block_bytes": (i64, [C.c_int]),
        "gq_profile_mmq_events": (None, [vp, vp]),
        "gq_dequant": (C.c_int, [C.c_int, vp, i64, i64, C.c_int, vp, vp]),
        "gq_linear_lora_fwd_workspace_size": (sz, [P(LoraLinear), i64]),
        "gq_linear_lora_fwd": (C.c_int, [P(LoraLinear), vp, i64, vp, vp, vp, sz, vp]),
        "gq_linear_lora_bwd_workspace_size": (sz, [P(LoraLinear), i64]),
        "gq_linear_lora_bwd": (C.c_int, [P(LoraLinear), vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "gq_noalloc_scratch_bytes": (sz, []),
        "gq_linear_lora_bwd_noalloc": (C.c_int, [P(LoraLinear), vp, vp, vp, i64, vp, vp, vp, vp]),
        "gq_moe_route_workspace_size": (sz, [i64, i32, i32]),
        "gq_moe_route": (C.c_int, [vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "gq_moe_route_bwd": (C.c_int, [vp, vp, vp, i64, i32, i32, vp, vp]),
        "gq_moe_combine_fwd": (C.c_int, [vp, vp, vp, i64, i32, i64, vp, vp]),
        "gq_moe_combine_bwd": (C.c_int, [vp, vp, i64, i32, i64, vp, vp]),
        "gq_grouped_mmq_lora_fwd_workspace_size": (sz, [P(LoraLinear), i32, i64]),
        "gq_grouped_mmq_lora_fwd": (C.c_int, [P(LoraLinear), i32, i32, P(GroupedFwdArgs), vp, sz, vp]),
        "gq_grouped_mmq_lora_bwd_workspace_size": (sz, [P(LoraLinear), i32, i32, i64]),
        "gq_grouped_mmq_lora_bwd": (C.c_int, [P(LoraLinear), i32, i32, P(GroupedBwdArgs), vp, sz, vp]),
        "gq_lmhead_chunked_ce_workspace_size": (sz, [P(LoraLinear), i64, i64]),
        "gq_lmhead_chunked_ce": (C.c_int, [P(LoraLinear), vp, vp, i64, i64, i64, f32, vp, vp, vp,
                                           vp, vp, vp, sz, vp]),
        "gq_rmsnorm_fwd": (C.c_int, [vp, vp, i64, i64, f32, vp, vp, vp]),
        "gq_rmsnorm_bwd": (C.c_int, [vp, vp, vp, vp, i64, i64, vp, vp]),
        "gq_adamw8bit_step": (C.c_int, [vp, vp, vp, vp, vp, vp, i64, i64, f32, f32, f32, f32, f32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def lib():
    return load_library()


def last_error() -> str:
    return lib().gq_last_error().decode()


def _check(rc: int):
    if rc != GQ_OK:
        raise GQError(rc, last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _expect(t, name: str, dtype, shape=None, min_rows=None, on_gpu=True):
    """Argument check before any pointer reaches the library: a contiguous
    GPU tensor of `dtype` with exactly `shape` (entries None: any size), or
    at least `min_rows` rows.  The C layer only sees raw pointers, so a wrong
    dtype, layout or size would otherwise be read as garbage or past the end
    of the allocation."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None:
        ok = t.dim() == len(shape) and all(s is None or int(a) == int(s) for a, s in zip(t.shape, shape))
        if not ok:
            want = tuple("*" if s is None else int(s) for s in shape)
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want}")
    if min_rows is not None and (t.dim() < 1 or t.shape[0] < min_rows):
        raise ValueError(f"{name}: {t.shape[0] if t.dim() else 0} rows, at least {min_rows} needed")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (row-major)")
    if on_gpu and not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (device {t.device})")
    return t


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


@dataclass
class Proj:
    """A quantised projection (or E stacked experts) with its LoRA adapter.
    blocks: uint8 [E?, n_out, n_in/32*bs]; A: fp32 [E?, r, n_in]; B: fp32 [E?, n_out, r]."""
    qtype: int
    n_out: int
    n_in: int
    blocks: torch.Tensor
    A: torch.Tensor
    B: torch.Tensor
    scale: float
    n_experts: int = 1

    @property
    def rank(self) -> int:
        return self.A.shape[-2]

    def check(self):
        """Shapes, dtypes and sizes of the blocks and adapters against
        (qtype, n_out, n_in, n_experts); raises before any library call."""
        if self.qtype not in BLOCK_BYTES:
            raise ValueError(f"unknown qtype {self.qtype}")
        if self.n_in % 32:
            raise ValueError(f"n_in {self.n_in} is not a multiple of 32")
        E = self.n_experts
        nbytes = E * self.n_out * (self.n_in // 32) * BLOCK_BYTES[self.qtype]
        _expect(self.blocks, "blocks", torch.uint8, on_gpu=False)
        if self.blocks.numel() != nbytes:
            raise ValueError(f"blocks: {self.blocks.numel()} bytes, expected {nbytes} "
                             f"({E} x {self.n_out} rows x {self.n_in // 32} blocks of {BLOCK_BYTES[self.qtype]} B)")
        r = self.A.shape[-2] if self.A.dim() >= 2 else 0
        if not 1 <= r <= 16:
            raise ValueError(f"A {tuple(self.A.shape)}: rank {r} not in [1, 16]")
        lead = (E,) if E > 1 or self.A.dim() == 3 else ()
        _expect(self.A, "A", torch.float32, lead + (r, self.n_in), on_gpu=False)
        _expect(self.B, "B", torch.float32, lead + (self.n_out, r), on_gpu=False)
        for name, t in (("blocks", self.blocks), ("A", self.A), ("B", self.B)):
            _expect(t, name, t.dtype)
        _same_device(self.blocks, self.A, self.B)
        return self

    def c(self) -> LoraLinear:
        return LoraLinear(self.qtype, self.rank, self.n_out, self.n_in, _ptr(self.blocks),
                          _ptr(self.A), _ptr(self.B), float(self.scale), self.n_experts)


# ------------------------------------------------------------------ entry points
def dequant(qtype: int, blocks: torch.Tensor, rows: int, cols: int, out_dtype=torch.float32):
    if qtype not in BLOCK_BYTES or cols % 32:
        raise ValueError(f"dequant: qtype {qtype} / cols {cols}")
    _expect(blocks, "blocks", torch.uint8, on_gpu=False)
    if blocks.numel() < rows * (cols // 32) * BLOCK_BYTES[qtype]:
        raise ValueError(f"blocks: {blocks.numel()} bytes, {rows * (cols // 32) * BLOCK_BYTES[qtype]} needed")
    _expect(blocks, "blocks", torch.uint8)
    out = torch.empty((rows, cols), dtype=out_dtype, device=blocks.device)
    code = F32 if out_dtype == torch.float32 else BF16
    _check(lib().gq_dequant(qtype, _ptr(blocks), rows, cols, code, _ptr(out), _stream()))
    return out


def linear_lora_fwd(p: Proj, x: torch.Tensor):
    p.check()
    _expect(x, "x", torch.bfloat16, (None, p.n_in))
    _same_device(x, p.blocks)
    T = x.shape[0]
    y = torch.empty((T, p.n_out), dtype=torch.bfloat16, device=x.device)
    xa = torch.empty((T, p.rank), dtype=torch.float32, device=x.device)
    L = p.c()
    nbytes = lib().gq_linear_lora_fwd_workspace_size(C.byref(L), T)
    ws = _workspace(nbytes, x.device)
    _check(lib().gq_linear_lora_fwd(C.byref(L), _ptr(x), T, _ptr(y), _ptr(xa), _ptr(ws), nbytes,
                                    _stream()))
    return y, xa


def _check_lin_bwd(p: Proj, x, xa, dy):
    p.check()
    _expect(x, "x", torch.bfloat16, (None, p.n_in))
    T = x.shape[0]
    _expect(xa, "xa", torch.float32, (T, p.rank))
    _expect(dy, "dy", torch.bfloat16, (T, p.n_out))
    _same_device(x, xa, dy, p.blocks)
    return T


def linear_lora_bwd(p: Proj, x, xa, dy, need_dx: bool = True, ws: torch.Tensor | None = None):
    T = _check_lin_bwd(p, x, xa, dy)
    if ws is not None:
        _expect(ws, "ws", torch.uint8)
    dx = torch.empty((T, p.n_in), dtype=torch.bfloat16, device=x.device) if need_dx else None
    dA = torch.empty((p.rank, p.n_in), dtype=torch.float32, device=x.device)
    dB = torch.empty((p.n_out, p.rank), dtype=torch.float32, device=x.device)
    L = p.c()
    nbytes = lib().gq_linear_lora_bwd_workspace_size(C.byref(L), T)
    if ws is None or ws.numel() < nbytes:
        ws = _workspace(nbytes, x.device)
    _check(lib().gq_linear_lora_bwd(C.byref(L), _ptr(x), _ptr(xa), _ptr(dy), T, _ptr(dx), _ptr(dA),
                                    _ptr(dB), _ptr(ws), nbytes, _stream()))
    return dx, dA, dB


def linear_lora_bwd_noalloc(p: Proj, x, xa, dy, dx=None, dA=None, dB=None):
    """gq_linear_lora_bwd_noalloc: the fast LoRA backward with the library's
    fixed device scratch (no workspace).  Outputs may be passed in
    (preallocated) so that the call itself allocates nothing."""
    T = _check_lin_bwd(p, x, xa, dy)
    if dx is None:
        dx = torch.empty((T, p.n_in), dtype=torch.bfloat16, device=x.device)
    if dA is None:
        dA = torch.empty((p.rank, p.n_in), dtype=torch.float32, device=x.device)
    if dB is None:
        dB = torch.empty((p.n_out, p.rank), dtype=torch.float32, device=x.device)
    _expect(dx, "dx", torch.bfloat16, (T, p.n_in))
    _expect(dA, "dA", torch.float32, (p.rank, p.n_in))
    _expect(dB, "dB", torch.float32, (p.n_out, p.rank))
    _same_device(x, dx, dA, dB)
    L = p.c()
    _check(lib().gq_linear_lora_bwd_noalloc(C.byref(L), _ptr(x), _ptr(xa), _ptr(dy), T, _ptr(dx),
                                            _ptr(dA), _ptr(dB), _stream()))
    return dx, dA, dB


def moe_route(logits: torch.Tensor, k: int):
    _expect(logits, "logits", torch.float32, (None, None))
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    sorted_ = torch.empty(T * k, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pos = torch.empty(T * k, dtype=torch.int32, device=dev)
    nbytes = lib().gq_moe_route_workspace_size(T, E, k)
    ws = _workspace(nbytes, dev)
    _check(lib().gq_moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _ptr(sorted_),
                              _ptr(offsets), _ptr(pos), _ptr(ws), nbytes, _stream()))
    return ids, w, sorted_, offsets, pos


def moe_route_bwd(ids, w, dw, E: int):
    _expect(ids, "ids", torch.int32, (None, None))
    T, k = ids.shape
    _expect(w, "w", torch.float32, (T, k))
    _expect(dw, "dw", torch.float32, (T, k))
    _same_device(ids, w, dw)
    dl = torch.empty((T, E), dtype=torch.float32, device=ids.device)
    _check(lib().gq_moe_route_bwd(_ptr(ids), _ptr(w), _ptr(dw), T, E, k, _ptr(dl), _stream()))
    return dl


def moe_combine_fwd(o, w, pos, T: int, k: int):
    _expect(o, "o", torch.bfloat16, (T * k, None))
    _expect(w, "w", torch.float32, None)
    _expect(pos, "pos", torch.int32, None)
    if w.numel() != T * k or pos.numel() != T * k:
        raise ValueError(f"w / pos: {w.numel()} / {pos.numel()} elements, expected {T * k}")
    _same_device(o, w, pos)
    H = o.shape[1]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=o.device)
    _check(lib().gq_moe_combine_fwd(_ptr(o), _ptr(w), _ptr(pos), T, k, H, _ptr(y), _stream()))
    return y


def moe_combine_bwd(dxrows, pos, T: int, k: int):
    _expect(dxrows, "dxrows", torch.bfloat16, (T * k, None))
    _expect(pos, "pos", torch.int32, (T * k,))
    _same_device(dxrows, pos)
    H = dxrows.shape[1]
    dx = torch.empty((T, H), dtype=torch.bfloat16, device=dxrows.device)
    _check(lib().gq_moe_combine_bwd(_ptr(dxrows), _ptr(pos), T, k, H, _ptr(dx), _stream()))
    return dx


def rmsnorm_fwd(x, w, eps: float = 1e-6):
    """y = x * rstd * w (bf16 [T, H]) and rstd (fp32 [T]); w fp32 [H]."""
    _expect(x, "x", torch.bfloat16, (None, None))
    T, H = x.shape
    _expect(w, "w", torch.float32, (H,))
    _same_device(x, w)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    rstd = torch.empty((T,), dtype=torch.float32, device=x.device)
    _check(lib().gq_rmsnorm_fwd(_ptr(x), _ptr(w), T, H, float(eps), _ptr(y), _ptr(rstd), _stream()))
    return y, rstd


def rmsnorm_bwd(dy, x, w, rstd):
    """Input gradient of rmsnorm_fwd (w is frozen)."""
    _expect(x, "x", torch.bfloat16, (None, None))
    T, H = x.shape
    _expect(dy, "dy", torch.bfloat16, (T, H))
    _expect(w, "w", torch.float32, (H,))
    _expect(rstd, "rstd", torch.float32, (T,))
    _same_device(x, dy, w, rstd)
    dx = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(lib().gq_rmsnorm_bwd(_ptr(dy), _ptr(x), _ptr(w), _ptr(rstd), T, H, _ptr(dx), _stream()))
    return dx


class AdamW8bitState:
    """8-bit AdamW states of one fp32 parameter tensor of n elements: codes
    uint8 [n] for m and v, one fp32 scale each per block of 256 (all zero =
    the initial state)."""

    def __init__(self, n: int, device):
        nb = (n + 255) // 256
        self.n = n
        self.step = 0
        self.m_codes = torch.zeros(n, dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros(n, dtype=torch.uint8, device=device)
        self.m_scale = torch.zeros(nb, dtype=torch.float32, device=device)
        self.v_scale = torch.zeros(nb, dtype=torch.float32, device=device)


def adamw8bit_step(p, g, st: AdamW8bitState, lr: float = 1e-4, betas=(0.9, 0.999), eps: float = 1e-8,
                   weight_decay: float = 0.0):
    """One in-place AdamW step of the fp32 tensor p (contiguous) with grad g."""
    _expect(p, "p", torch.float32, None)
    _expect(g, "g", torch.float32, None)
    if p.numel() != st.n or g.numel() != st.n:
        raise ValueError(f"p / g: {p.numel()} / {g.numel()} elements, the state holds {st.n}")
    _same_device(p, g, st.m_codes)
    st.step += 1
    _check(lib().gq_adamw8bit_step(_ptr(p), _ptr(g), _ptr(st.m_codes), _ptr(st.v_codes),
                                   _ptr(st.m_scale), _ptr(st.v_scale), st.n, st.step, float(lr),
                                   float(betas[0]), float(betas[1]), float(eps), float(weight_decay),
                                   _stream()))


def _projs(ps):
    arr = (LoraLinear * len(ps))(*[p.c() for p in ps])
    return arr


def _check_group(projs, offsets, M: int, gather):
    for p in projs:
        p.check()
    E = projs[0].n_experts
    _expect(offsets, "offsets", torch.int32, (E + 1,))
    if gather is not None:
        _expect(gather, "gather", torch.int32, (M,))
    _same_device(offsets, gather, *[p.blocks for p in projs])


def grouped_mmq_lora_fwd(projs, epilogue: int, inp, gather, gather_div: int, offsets, M: int, ws=None):
    """Grouped forward; `ws` (uint8, optional) is the workspace to use, whose
    first 32-bit word reports inconsistent offsets after synchronising."""
    _check_group(projs, offsets, M, gather)
    _expect(inp, "inp", torch.bfloat16, (None, projs[0].n_in), min_rows=None if gather is not None else M)
    dev = inp.device
    N = projs[0].n_out
    r = projs[0].rank
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    g = u = None
    if epilogue == EPI_SWIGLU:
        g = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        u = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    xa = torch.empty((len(projs), M, r), dtype=torch.float32, device=dev)
    arr = _projs(projs)
    nbytes = lib().gq_grouped_mmq_lora_fwd_workspace_size(arr, len(projs), M)
    if ws is None or ws.numel() < nbytes:
        ws = _workspace(nbytes, dev)
    else:
        _expect(ws, "ws", torch.uint8, None)
    a = GroupedFwdArgs(_ptr(inp), _ptr(gather), gather_div, _ptr(offsets), M, _ptr(out), _ptr(g),
                       _ptr(u), _ptr(xa))
    _check(lib().gq_grouped_mmq_lora_fwd(arr, len(projs), epilogue, C.byref(a), _ptr(ws), nbytes,
                                         _stream()))
    return out, g, u, xa


def grouped_mmq_lora_bwd(projs, mode: int, **t):
    """Thin wrapper: `t` maps gq_grouped_bwd_args field names to tensors/ints."""
    M = int(t["M"])
    _check_group(projs, t["offsets"], M, t.get("gather"))
    H = projs[0].n_out if mode == BWD_DOWN_SWIGLU else projs[0].n_in
    I = projs[0].n_in if mode == BWD_DOWN_SWIGLU else projs[0].n_out
    E, r = projs[0].n_experts, projs[0].rank
    gathered = t.get("gather") is not None
    want = {"dy": (torch.bfloat16, (None, H)), "x": (torch.bfloat16, (None, H)),
            "w_flat": (torch.float32, (M,)), "sorted": (torch.int32, (M,)),
            "g": (torch.bfloat16, (M, I)), "u": (torch.bfloat16, (M, I)), "h": (torch.bfloat16, (M, I)),
            "xa_d": (torch.float32, (M, r)), "dw_flat": (torch.float32, (M,)),
            "dA_d": (torch.float32, (E, r, I)), "dB_d": (torch.float32, (E, H, r)),
            "dg": (torch.bfloat16, (M, I)), "du": (torch.bfloat16, (M, I)),
            "dgB": (torch.float32, (M, r)), "duB": (torch.float32, (M, r)),
            "xa": (torch.float32, (2, M, r)), "dxrows": (torch.bfloat16, (M, H)),
            "dA_g": (torch.float32, (E, r, H)), "dB_g": (torch.float32, (E, I, r)),
            "dA_u": (torch.float32, (E, r, H)), "dB_u": (torch.float32, (E, I, r))}
    for name, (dt, shape) in want.items():
        v = t.get(name)
        if v is None:
            continue
        if name in ("w_flat", "dw_flat", "sorted"):  # flat [M] views of [T, k] arrays
            _expect(v, name, dt, None)
            if v.numel() != M:
                raise ValueError(f"{name}: {v.numel()} elements, expected {M}")
        else:
            _expect(v, name, dt, shape, min_rows=None if gathered or name not in ("dy", "x") else M)
    arr = _projs(projs)
    dev = t["offsets"].device
    nbytes = lib().gq_grouped_mmq_lora_bwd_workspace_size(arr, len(projs), mode, M)
    ws = t.pop("ws", None)
    if ws is None or ws.numel() < nbytes:
        ws = _workspace(nbytes, dev)
    a = GroupedBwdArgs()
    for name, _ in GroupedBwdArgs._fields_:
        v = t.get(name)
        if v is None:
            continue
        setattr(a, name, v if isinstance(v, int) else _ptr(v))
    if not t.get("gather_div"):
        a.gather_div = 1
    _check(lib().gq_grouped_mmq_lora_bwd(arr, len(projs), mode, C.byref(a), _ptr(ws), nbytes,
                                         _stream()))


def lmhead_chunked_ce(head: Proj, h, labels, chunk_rows: int = 4096, ignore_index: int = -100,
                      grad_scale: float = 1.0, want_grad: bool = True, ws=None):
    head.check()
    _expect(h, "h", torch.bfloat16, (None, head.n_in))
    T = h.shape[0]
    _expect(labels, "labels", torch.int64, (T,))
    _same_device(h, labels, head.blocks)
    dev = h.device
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    dh = dA = dB = None
    if want_grad:
        dh = torch.empty((T, head.n_in), dtype=torch.bfloat16, device=dev)
        dA = torch.empty((head.rank, head.n_in), dtype=torch.float32, device=dev)
        dB = torch.empty((head.n_out, head.rank), dtype=torch.float32, device=dev)
    L = head.c()
    nbytes = lib().gq_lmhead_chunked_ce_workspace_size(C.byref(L), T, chunk_rows)
    if ws is None or ws.numel() < nbytes:
        ws = _workspace(nbytes, dev)
    _check(lib().gq_lmhead_chunked_ce(C.byref(L), _ptr(h), _ptr(labels), T, chunk_rows,
                                      ignore_index, grad_scale, _ptr(loss), _ptr(lse), _ptr(dh),
                                      _ptr(dA), _ptr(dB), _ptr(ws), nbytes, _stream()))
    return dict(loss=loss, lse=lse, dh=dh, dA=dA, dB=dB, ws=ws)


# ------------------------------------------------------------ MoE layer helpers
@dataclass
class MoEWeights:
    gate: Proj
    up: Proj
    down: Proj


def moe_ffn_fwd(wts: MoEWeights, x, logits, k: int):
    """Routed SwiGLU expert FFN forward: routing, grouped gate/up MMQ with the
    SwiGLU epilogue, grouped down MMQ, combine.  Returns y and the saved state."""
    T = x.shape[0]
    ids, w, sorted_, offsets, pos = moe_route(logits, k)
    M = T * k
    h, g, u, xa_gu = grouped_mmq_lora_fwd([wts.gate, wts.up], EPI_SWIGLU, x, sorted_, k, offsets, M)
    o, _, _, xa_d = grouped_mmq_lora_fwd([wts.down], EPI_NONE, h, None, 1, offsets, M)
    y = moe_combine_fwd(o, w, pos, T, k)
    saved = dict(ids=ids, w=w, sorted=sorted_, offsets=offsets, pos=pos, g=g, u=u, h=h,
                 xa_gu=xa_gu, xa_d=xa_d[0], o=o)
    return y, saved


def moe_ffn_bwd(wts: MoEWeights, x, dy, saved, k: int, E: int):
    """Backward of moe_ffn_fwd: returns dx, dlogits and the adapter gradients."""
    T, H = x.shape
    M = T * k
    I = wts.gate.n_out
    r = wts.gate.rank
    dev = x.device
    f32, bf = torch.float32, torch.bfloat16
    dg = torch.empty((M, I), dtype=bf, device=dev)
    du = torch.empty((M, I), dtype=bf, device=dev)
    dgB = torch.empty((M, r), dtype=f32, device=dev)
    duB = torch.empty((M, r), dtype=f32, device=dev)
    dw_flat = torch.empty(M, dtype=f32, device=dev)
    grads = dict(dA_d=torch.empty((E, r, I), dtype=f32, device=dev),
                 dB_d=torch.empty((E, H, r), dtype=f32, device=dev),
                 dA_g=torch.empty((E, r, H), dtype=f32, device=dev),
                 dB_g=torch.empty((E, I, r), dtype=f32, device=dev),
                 dA_u=torch.empty((E, r, H), dtype=f32, device=dev),
                 dB_u=torch.empty((E, I, r), dtype=f32, device=dev))
    grouped_mmq_lora_bwd([wts.down, wts.gate, wts.up], BWD_DOWN_SWIGLU, offsets=saved["offsets"],
                         M=M, gather=saved["sorted"], gather_div=k, dy=dy, w_flat=saved["w"],
                         sorted=saved["sorted"], g=saved["g"], u=saved["u"], h=saved["h"],
                         xa_d=saved["xa_d"], dw_flat=dw_flat, dA_d=grads["dA_d"],
                         dB_d=grads["dB_d"], dg=dg, du=du, dgB=dgB, duB=duB)
    dxrows = torch.empty((M, H), dtype=bf, device=dev)
    grouped_mmq_lora_bwd([wts.gate, wts.up], BWD_GATEUP, offsets=saved["offsets"], M=M,
                         gather=saved["sorted"], gather_div=k, x=x, xa=saved["xa_gu"], dg=dg,
                         du=du, dgB=dgB, duB=duB, dxrows=dxrows, dA_g=grads["dA_g"],
                         dB_g=grads["dB_g"], dA_u=grads["dA_u"], dB_u=grads["dB_u"])
    dx = moe_combine_bwd(dxrows, saved["pos"], T, k)
    dlogits = moe_route_bwd(saved["ids"], saved["w"], dw_flat.view(T, k), E)
    return dict(dx=dx, dlogits=dlogits, dw=dw_flat.view(T, k), dg=dg, du=du, **grads)
