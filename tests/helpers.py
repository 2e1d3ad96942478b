"""Shared test helpers: comparisons and torch <-> numpy plumbing (no method arithmetic)."""
from __future__ import annotations

import numpy as np
import torch


def np64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    return t.numpy().astype(np.float64)


def normwise(x, ref) -> float:
    """max |x - ref| / max |ref| (normwise relative error of one output tensor)."""
    x, ref = np64(x), np64(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)


def assert_close(name, x, ref, tol):
    e = normwise(x, ref)
    assert np.isfinite(e) and e <= tol, f"{name}: normwise error {e:.3e} > {tol:.1e}"
    return e
