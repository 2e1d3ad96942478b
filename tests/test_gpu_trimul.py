"""GPU parity of the triangular multiplicative update (include/tri_mul.h) against the fp64 oracle
(oracle/trimul.py), both edge directions, forward and backward, through the C ABI.

Bar: normwise max|x - ref| / max|ref| <= 2e-2 per output tensor (bf16 inputs and outputs, fp32 accumulation),
for y, dz and every parameter gradient.  Sizes: ragged ones (1, 5, 37, 100, 130: tiles of the 128-wide GEMMs and
of the 64-pair per-pair kernels cut off), the crops 384 and 768, and 5-run bitwise repeats.
"""
from __future__ import annotations

import sys

import pytest
import torch

from oracle import trimul as TM
import triangle_attention_tri_amd as ta
from triangle_attention_tri_amd import inputs
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu
TOL = 2e-2
GRADS = ("dz", "dgamma_in", "dbeta_in", "dw_in", "dgamma_out", "dbeta_out", "dw_out")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(x, device, incoming):
    xd = {k: v.to(device) for k, v in x.items()}
    y, saved = ta.trimul_fwd(xd["z"], xd, incoming)
    g = ta.trimul_bwd(xd["z"], xd, saved, xd["dy"], incoming)
    torch.cuda.synchronize()
    return dict(y=y, **g)


def compare(name, x, got, incoming):
    ref = TM.trimul_bwd(x["z"], x["gamma_in"], x["beta_in"], x["w_in"], x["gamma_out"], x["beta_out"], x["w_out"],
                        x["dy"], incoming=incoming)
    errs = {"y": assert_close(f"{name}:y", got["y"].cpu(), ref["y"], TOL)}
    for key in GRADS:
        errs[key] = assert_close(f"{name}:{key}", got[key].cpu(), ref[key], TOL)
    log(name, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("incoming", [False, True])
@pytest.mark.parametrize("n", [1, 5, 37, 100, 130])
def test_trimul_small(device, n, incoming):
    log(f"trimul n={n} incoming={incoming}")
    x = inputs.trimul_inputs(n, seed=70 + n)
    compare(f"trimul{n}:{'in' if incoming else 'out'}", x, run(x, device, incoming), incoming)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("incoming", [False, True])
@pytest.mark.parametrize("n", [384, 768])
def test_trimul_crops(device, n, incoming):
    """The crop sizes the pages train at, every element of every output."""
    log(f"trimul n={n} incoming={incoming}")
    x = inputs.trimul_inputs(n, seed=n)
    got = {k: v.cpu() for k, v in run(x, device, incoming).items()}
    torch.cuda.empty_cache()
    compare(f"trimul{n}:{'in' if incoming else 'out'}", x, got, incoming)


@pytest.mark.parametrize("incoming", [False, True])
def test_trimul_repeat(device, incoming):
    """Five calls with fresh output buffers are bitwise identical (fixed-order weight-gradient sums)."""
    x = inputs.trimul_inputs(256, seed=3)
    first = run(x, device, incoming)
    for rep in range(4):
        again = run(x, device, incoming)
        for k in first:
            assert torch.equal(first[k], again[k]), f"run {rep + 1}: {k} differs"
