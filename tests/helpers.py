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


MASK_LOGIT = -1e9  # value a masked logit is replaced by (the forward's reading of the key mask)


def assert_lse(name, x, ref, tol_abs):
    """Log-sum-exp [rows, H, nq] against the fp64 reference, element by element.

    A row that keeps at least one key has |lse| of order log n plus the logit
    scale, so it is checked with an absolute bound: a normwise bound would be
    scaled by the largest |lse| of the tensor, which a fully masked row puts near
    1e9.  A fully masked row (reference MASK_LOGIT + log n) must hold that value
    rounded to float32 exactly.
    """
    x, ref = np64(x), np64(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    dead = ref < 0.5 * MASK_LOGIT
    live = ~dead
    err = float(np.max(np.abs(x[live] - ref[live]))) if live.any() else 0.0
    assert np.isfinite(err) and err <= tol_abs, f"{name}: max |lse - ref| {err:.3e} > {tol_abs:.1e}"
    if dead.any():
        want = ref[dead].astype(np.float32).astype(np.float64)
        assert np.array_equal(x[dead], want), f"{name}: fully masked rows' lse differ from MASK_LOGIT + log n"
    return err


def lse_tol(tol):
    """Absolute log-sum-exp bound that goes with a normwise bound: fp32 runs 1e-4, bf16 runs 2e-2."""
    return 1e-4 if tol <= 1e-4 else 2e-2
