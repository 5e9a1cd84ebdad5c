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


def bf16_rounding(want: np.ndarray) -> np.ndarray:
    """|want - bf16(want)|: the error any bf16 output of the exact value carries
    (round to nearest even, through float32)."""
    import workloads as W
    w = np.asarray(want, dtype=np.float64)
    r = W.bf16_bits_to_f32(W.f32_to_bf16_bits(w.astype(np.float32))).astype(np.float64)
    out = np.abs(w - r)
    out[~np.isfinite(w)] = 0.0
    return out


def check_bf16_out(name: str, got, want, tol: float, net_from: float = 2.0):
    """Max-abs check of a bf16 output against the fp64 oracle.

    Every element whose exact value has |want| < net_from must meet the raw
    bound |got - want| <= tol.  An element with |want| >= net_from is held to
    the same tol net of its own bf16 rounding |want - bf16(want)|: there the
    output's half-ulp (2^-7 in [2, 4), 2^-6 in [4, 8)) plus the bf16 rounding
    of the probabilities before the matrix product (up to 2^-9 |want|) can
    exceed 1e-2 with nothing wrong (e.g. O = V_0 on the first causal rows).
    Prints the raw maximum and how many elements took the net rule."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = max_abs_err(got, want)
    assert np.isfinite(err), f"{name}: non-finite pattern or infinite values differ"
    fin = np.isfinite(want)
    diff = np.abs(got - want)
    big = fin & (np.abs(want) >= net_from)
    small = fin & ~big
    err_small = float(np.max(diff[small])) if small.any() else 0.0
    err_net = float(np.max(diff[big] - bf16_rounding(want[big]))) if big.any() else 0.0
    err_big_raw = float(np.max(diff[big])) if big.any() else 0.0
    say(f"    {name}: max|err| = {err:.3e}; |want| < {net_from:g}: {err_small:.3e} raw (tol {tol:.0e}); "
        f"{int(big.sum())} elements with |want| >= {net_from:g}: raw {err_big_raw:.3e}, "
        f"net of bf16 output rounding {err_net:.3e} (tol {tol:.0e})")
    assert err_small <= tol, f"{name}: max abs error {err_small:.3e} > {tol:.1e} where |want| < {net_from:g}"
    assert err_net <= tol, f"{name}: error net of output rounding {err_net:.3e} > {tol:.1e} where |want| >= {net_from:g}"
    return max(err_small, err_net)


def check(name: str, got, want, tol: float, extra: str = ""):
    err = max_abs_err(got, want)
    say(f"    {name}: max|err| = {err:.3e} (tol {tol:.0e}) {extra}")
    assert err <= tol, f"{name}: max abs error {err:.3e} > {tol:.1e} {extra}"
    return err
