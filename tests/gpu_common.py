"""Helpers shared by the GPU parity tests: device transfer and the tolerance.

Tolerance (the max-relative bound of the bf16 sublayer with an fp32 state):
    err = max_i |got_i - ref_i| / max_i |ref_i|
must be <= 2e-3 for bf16 inputs with fp32 state, <= 1e-5 for the fp32 path.
Where the library stores bf16, one bf16 ulp of |ref_i| (2^-7 |ref_i| bounds
it) is allowed on top, element by element.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda"
TOL_BF16 = 2e-3
TOL_F32 = 1e-5


def dev(a, bf16: bool = False) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    denom = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (denom if denom > 0 else 1.0)


def check(got, ref, tol: float, what: str, stored_bf16: bool = False) -> float:
    """Assert the max-relative bound; returns the measured metric."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    denom = float(np.max(np.abs(ref))) if ref.size else 1.0
    allow = tol * denom + (np.abs(ref) * 2.0 ** -7 if stored_bf16 else 0.0)
    err = np.abs(got - ref)
    bad = err > allow
    metric = max_rel(got, ref)
    print(f"[parity] {what}: max-rel {metric:.3e} (bound {tol:.0e}{' + 1 bf16 ulp' if stored_bf16 else ''})",
          file=sys.stderr, flush=True)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements out of bound; "
                           f"worst |err| {err.max():.3e} vs bound {tol * denom:.3e}")
    return metric


def worst_ratio(got, ref, tol: float) -> float:
    """Worst element's error divided by the bound (the golden PR's negative-control statistic)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / (tol * np.max(np.abs(ref))))
