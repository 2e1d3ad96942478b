"""GPU: rounding-residual compensation of the saved attention (tri_attn_fwd_rc / tri_attn_bwd_rc).

The compensated pair must meet the same bar as the plain one against the fp64
oracle, leave the forward outputs and dv bit for bit unchanged, and carry a
residual that brings the saved attention closer to the exact value.  On these
seeded inputs it lowers the mean error of dgate by more than 10% and does not
raise that of dq, dk or dbias (measured reductions there are 0.5-1%; the pages
report 28-47% for their kernels, whose other bf16 error sources evidently
differ).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import triangle_attention_tri_amd as ta
from triangle_attention_tri_amd import inputs
from tests.helpers import assert_close, np64
from tests.test_gpu_parity import log, to_dev

pytestmark = pytest.mark.gpu

KEYS = ("dq", "dk", "dv", "dbias", "dgate")


def mean_rel(x, ref):
    x, ref = np64(x), np64(ref)
    return float(np.mean(np.abs(x - ref)) / np.mean(np.abs(ref)))


def decode(attn_bf16, codes):
    """The header's definition: ab + code * 2^(e - 142), e the biased exponent of ab (1 for zero/subnormal)."""
    ab = attn_bf16.float().cpu()
    e = ((ab.view(torch.int32) >> 23) & 0xFF).numpy()
    e = np.where(e == 0, 1, e)
    return ab.numpy().astype(np.float64) + codes.cpu().numpy().astype(np.float64) * np.exp2(e - 142.0)


@pytest.mark.parametrize("widx", [1, 2])
def test_residual_compensation(device, widx):
    w = inputs.WORKLOADS[widx]
    log(f"residual compensation, workload {widx} {w.name}")
    xc = inputs.workload_inputs(widx)
    x = to_dev(xc, device)
    args = (x["q"], x["k"], x["v"], x["bias"], x["gate"], x["mask"])
    out, attn, lse, res = ta.fwd(*args, residual=True)
    out0, attn0, lse0 = ta.fwd(*args)
    g0 = dict(zip(KEYS, ta.bwd(*args, attn0, lse0, x["dout"])))
    g1 = dict(zip(KEYS, ta.bwd(*args, attn, lse, x["dout"], attn_residual=res)))
    g2 = dict(zip(KEYS, ta.bwd(*args, attn, lse, x["dout"], attn_residual=res)))
    torch.cuda.synchronize()
    # the bf16 outputs are those of the plain forward; dv does not depend on D
    assert torch.equal(out, out0) and torch.equal(attn, attn0) and torch.equal(lse, lse0)
    assert torch.equal(g1["dv"], g0["dv"])
    for k in KEYS:
        assert torch.equal(g1[k], g2[k]), f"{k} differs between repeated compensated calls"
    ref = oracle.attn_bwd(xc["q"], xc["k"], xc["v"], xc["bias"], xc["gate"], xc["mask"], xc["dout"])
    for k in KEYS:
        assert_close(f"rc:{k}", g1[k], ref[k], w.tol)
    # the residual codes use their range and bring attn closer to the exact value
    codes = res.cpu().numpy()
    assert codes.min() >= -127 and codes.max() <= 127 and np.count_nonzero(codes) > codes.size // 2
    aref = np64(ref["attn"])
    e_bf16 = np.max(np.abs(np64(attn) - aref)) / np.max(np.abs(aref))
    e_comp = np.max(np.abs(decode(attn, res) - aref)) / np.max(np.abs(aref))
    gains = {k: 1.0 - mean_rel(g1[k], ref[k]) / mean_rel(g0[k], ref[k]) for k in KEYS}
    log(f"  attn error bf16 {e_bf16:.3e}, compensated {e_comp:.3e}; mean-error reduction "
        + " ".join(f"{k}={100 * v:+.1f}%" for k, v in gains.items()))
    assert e_comp < 0.6 * e_bf16
    assert gains["dgate"] > 0.10
    for k in ("dq", "dk", "dbias"):
        assert gains[k] >= 0.0, f"{k}: compensated mean error above the plain one"


def test_residual_ending_node_masked(device):
    """The compensated pair at the ending node with a mask that drops a whole row: same bar as the
    plain pair, dv and the forward outputs unchanged."""
    from tests.test_gpu_parity import check_full, TOL
    n = 45
    xc = inputs.attn_inputs(n, 4, 32, torch.bfloat16, seed=7, bias_std=2.0)
    xc["mask"] = inputs.random_mask(n, seed=9, p_keep=0.8, full_rows=(4,))
    x = to_dev(xc, device)
    args = (x["q"], x["k"], x["v"], x["bias"], x["gate"], x["mask"])
    out, attn, lse, res = ta.fwd(*args, ending=True, residual=True)
    out0, attn0, lse0 = ta.fwd(*args, ending=True)
    assert torch.equal(out, out0) and torch.equal(attn, attn0) and torch.equal(lse, lse0)
    g0 = ta.bwd(*args, attn0, lse0, x["dout"], ending=True)
    g1 = ta.bwd(*args, attn, lse, x["dout"], ending=True, attn_residual=res)
    torch.cuda.synchronize()
    assert torch.equal(g1[2], g0[2])
    got = dict(out=out, attn=attn, lse=lse, dq=g1[0], dk=g1[1], dv=g1[2], dbias=g1[3], dgate=g1[4])
    check_full(f"rc_end{n}", xc, got, TOL[torch.bfloat16], ending=True)
