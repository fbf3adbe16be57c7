"""Helpers for the GPU parity tests: move seeded numpy inputs to the device, read results
back, and compare them with the oracle under the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import pytest

TOL_F32 = 1e-5          # fp32 path, and int8-KV against the dequantized oracle with fp32 output
TOL_BF16 = 1e-2         # bf16 output on unit-variance inputs
TOL_E2E = 5e-3          # int8-KV end to end against unquantized attention


def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str):
    """numpy -> device tensor.  dtype 'bf16' requires values already representable in bf16."""
    torch = torch_gpu()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        tb = t.to(torch.bfloat16)
        assert torch.equal(tb.float(), t.float()), "values are not bf16-representable"
        return tb.cuda()
    if dtype == "f32":
        return t.float().cuda()
    if dtype == "i8":
        return t.to(torch.int8).cuda()
    raise ValueError(dtype)


def to_np(t) -> np.ndarray:
    torch = torch_gpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |ref| (the largest rounding error of a correctly rounded bf16 store)."""
    a = np.abs(ref).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def check_close(out: np.ndarray, ref: np.ndarray, tol: float, what: str, mask=None):
    diff = np.abs(out.astype(np.float64) - ref)
    if mask is not None:
        diff = np.where(mask, diff, 0.0)
    assert np.all(np.isfinite(out[mask] if mask is not None else out)), f"{what}: non-finite output"
    m = float(diff.max()) if diff.size else 0.0
    say(f"  {what}: max abs err {m:.3e} (tol {tol:.1e})")
    assert m <= tol, f"{what}: max abs err {m:.3e} > {tol:.1e}"
    return m


def check_bf16_output(out: np.ndarray, ref: np.ndarray, what: str):
    """bf16 outputs: every element within 1e-2 of the oracle, except that an element whose
    correctly rounded bf16 value alone is further than 1e-2 away (|ref| >= 4) may differ by its
    rounding plus a 6e-3 kernel allowance.  The raw max and the count above 1e-2 are printed."""
    diff = np.abs(out.astype(np.float64) - ref)
    hu = bf16_half_ulp(ref)
    bound = np.where(hu > TOL_BF16, hu + 6e-3, TOL_BF16)
    m = float(diff.max()) if diff.size else 0.0
    n_over = int((diff > TOL_BF16).sum())
    say(f"  {what}: max abs err {m:.3e}, {n_over} elements > 1e-2, max(err - half ulp) "
        f"{float((diff - hu).max()) if diff.size else 0.0:.3e}")
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    assert np.all(diff <= bound), f"{what}: error beyond the bf16 bound (max {m:.3e})"
    return m
