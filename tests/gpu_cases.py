"""Helpers shared by the GPU tests: device transfer, the oracle comparison, tolerances.

Tolerances (max-abs against the fp64 oracle):
  bf16 path: O <= 1e-2, lse <= 1e-3, dQ/dK/dV <= 2e-2
  fp32 path: O, lse, dQ/dK/dV <= 1e-5
"""
from __future__ import annotations

import sys

import numpy as np

TOL_BF16 = {"o": 1e-2, "lse": 1e-3, "dq": 2e-2, "dk": 2e-2, "dv": 2e-2}
TOL_F32 = {"o": 1e-5, "lse": 1e-5, "dq": 1e-5, "dk": 1e-5, "dv": 1e-5}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(t, dtype: str):
    """A workloads.Tensor (or float32 ndarray for f32) -> torch tensor on cuda:0."""
    import torch
    if dtype == "bf16":
        bits = np.ascontiguousarray(t.bits if hasattr(t, "bits") else t).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to("cuda:0")
    vals = t.values if hasattr(t, "values") else t
    return torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).to("cuda:0")


def to_host64(x) -> np.ndarray:
    import torch
    return x.detach().to(torch.float64).cpu().numpy()


def max_abs_err(got: np.ndarray, want: np.ndarray) -> float:
    """Max |got - want|; infinities must match exactly (e.g. lse of an empty row)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    fin = np.isfinite(want)
    if not np.array_equal(np.isfinite(got), fin):
        return float("inf")
    if not np.array_equal(got[~fin], want[~fin]):
        return float("inf")
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(got[fin] - want[fin])))


def check(name: str, got, want, tol: float, extra: str = ""):
    err = max_abs_err(got, want)
    say(f"    {name}: max|err| = {err:.3e} (tol {tol:.0e}) {extra}")
    assert err <= tol, f"{name}: max abs error {err:.3e} > {tol:.1e} {extra}"
    return err
