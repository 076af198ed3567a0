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
