"""Shared helpers of the GPU parity tests: host <-> device marshalling of the
seeded inputs and the comparison metrics (no method arithmetic here)."""
import numpy as np
import torch

DEV = "cuda"
TOL = 1e-2  # relative Frobenius error bar for floating-point outputs


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def i64_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(DEV)


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.array(a, dtype=np.uint8, order="C", copy=True)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def rel_frob(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite values in GPU output"
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return float(np.abs(got).max()) if got.size else 0.0
    return float(np.linalg.norm(got - ref) / nr)


def check(name, got, ref, tol=TOL):
    e = rel_frob(got, ref)
    assert e <= tol, f"{name}: relative Frobenius error {e:.3e} > {tol}"
    return e


def same_f32_bits(got: np.ndarray, exp: np.ndarray):
    """Bit-exact float comparison with +0 == -0 and NaN positions equal."""
    got = np.asarray(got, np.float32)
    exp = np.asarray(exp, np.float32)
    assert got.shape == exp.shape
    ng, ne = np.isnan(got), np.isnan(exp)
    assert np.array_equal(ng, ne)
    ok = ~ne
    bad = np.nonzero(got[ok] != exp[ok])[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {got[ok][bad[:4]]} vs {exp[ok][bad[:4]]}"


# Per-expert bar for the adapter gradients.  An expert with a handful of
# rows does not average the bf16 rounding of its decoded weights (the MFMA
# operands) and of the stored g, u, dg over many rows, so one row's rank-r
# gradient carries that rounding almost undiluted.  A float64 emulation of
# the bf16 rounding points (decoded weights in the forward and backward
# MMQ, stored g, u, dg) reproduces the GPU's per-expert errors to three
# digits: 1.09e-2 for the single-row expert 124 of the 2-bit Zipf workload,
# 2.54e-2 for the single-row expert 2 of the Q4_0 layer at 16 tokens.  The
# bar is therefore the tensor bar for experts with 32 rows or more and grows
# as 1/sqrt(rows) below that (5.7e-2 for one row); a broken path (wrong row,
# wrong expert, missing term) errs by O(1) and still fails.
ROWS_FULL_BAR = 32


def check_per_expert(name, got, ref, rows, tol=TOL):
    """Relative Frobenius error per expert (leading axis) against
    tol * max(1, sqrt(32 / rows_e)) for every expert whose reference is
    non-zero; exact zeros where it is zero.  Returns the largest error
    divided by its expert's bar."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rows = np.asarray(rows)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    worst = 0.0
    for e in range(ref.shape[0]):
        nr = np.linalg.norm(ref[e])
        if nr == 0.0:
            assert np.all(got[e] == 0.0), f"{name}[{e}]: reference is zero, got non-zeros"
            continue
        bar = tol * max(1.0, float(np.sqrt(ROWS_FULL_BAR / max(int(rows[e]), 1))))
        err = float(np.linalg.norm(got[e] - ref[e]) / nr)
        assert err <= bar, f"{name}[{e}] ({rows[e]} rows): relative Frobenius error {err:.3e} > {bar:.3e}"
        worst = max(worst, err / bar)
    return worst


class GuardedTorch:
    """Stands in for the ``torch`` module inside the binding during a GPU
    test: ``torch.empty`` / ``torch.zeros`` on the GPU return views into a
    larger buffer whose margins (GUARD bytes before and after) hold a fixed
    byte pattern.  ``check()`` synchronises and verifies that no margin byte
    changed, i.e. no kernel wrote outside the output or workspace it was
    given.  Everything else is the real torch.  Allocations made while a
    stream is being captured into a graph are passed through unguarded (the
    pattern fill would become part of the graph)."""

    GUARD = 4096
    PATTERN = 0xA5
    HOLD_BYTES = 8 << 30  # check and release held buffers beyond this

    def __init__(self, real, device_types=("cuda",)):
        self._t = real
        self._types = tuple(device_types)
        self._held = []
        self._held_bytes = 0
        self.checked = 0

    def __getattr__(self, name):
        return getattr(self._t, name)

    def _alloc(self, size, dtype, device, zero, kw):
        t = self._t
        if len(size) == 1 and isinstance(size[0], (tuple, list, t.Size)):
            size = tuple(size[0])
        size = tuple(int(s) for s in size)
        dev = t.device(device) if device is not None else None
        if (dev is None or dev.type not in self._types or kw
                or (dev.type == "cuda" and t.cuda.is_current_stream_capturing())):
            f = t.zeros if zero else t.empty
            return f(size, dtype=dtype, device=device, **kw)
        dtype = dtype or t.get_default_dtype()
        esz = t.empty(0, dtype=dtype).element_size()
        n = 1
        for s in size:
            n *= s
        nbytes = n * esz
        G = self.GUARD
        raw = t.empty(nbytes + 2 * G, dtype=t.uint8, device=dev)
        raw[:G].fill_(self.PATTERN)
        raw[G + nbytes:].fill_(self.PATTERN)
        mid = raw[G:G + nbytes]
        if zero:
            mid.zero_()
        out = mid.view(dtype).view(size)
        self._held.append((raw, nbytes))
        self._held_bytes += raw.numel()
        if self._held_bytes > self.HOLD_BYTES:
            self.check()
        return out

    def empty(self, *size, dtype=None, device=None, **kw):
        return self._alloc(size, dtype, device, False, kw)

    def zeros(self, *size, dtype=None, device=None, **kw):
        return self._alloc(size, dtype, device, True, kw)

    def check(self):
        """Raise AssertionError if any guard byte of a held buffer changed;
        release the held buffers."""
        if not self._held:
            return
        t = self._t
        if any(raw.is_cuda for raw, _ in self._held):
            t.cuda.synchronize()
        G = self.GUARD
        bad = []
        for raw, nbytes in self._held:
            lo = raw[:G]
            hi = raw[G + nbytes:]
            nlo = int((lo != self.PATTERN).sum().item())
            nhi = int((hi != self.PATTERN).sum().item())
            if nlo or nhi:
                bad.append(f"buffer of {nbytes} bytes: {nlo} bytes changed before it, {nhi} after it")
        self.checked += len(self._held)
        self._held = []
        self._held_bytes = 0
        assert not bad, "writes outside an output or workspace: " + "; ".join(bad)
