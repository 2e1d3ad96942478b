"""Pins of the block oracle (LayerNorm + projections + attention + output linear).

Each test ties oracle/block.py to something other than its own arithmetic:
torch's float64 layer_norm / linear / autograd (library routines), central
finite differences, closed forms of the LayerNorm, identity weights that expose
the output layouts element by element, and the pair-transpose identity of the
ending node.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import block as B
from triangle_attention_tri_amd import inputs

H, C, CZ = 4, 32, 128


def params(n, seed, affine=True, cz=CZ):
    x = inputs.block_inputs(n, cz=cz, h=H, c=C, dtype=torch.float32, seed=seed, affine=affine)
    return {k: v.double() for k, v in x.items()}


def torch_block(x, ending, mask=None):
    """The block written with torch's own layer_norm / linear, autograd-ready, float64."""
    z = x["z"]
    n = z.shape[0]
    if ending:
        z = z.transpose(0, 1)
    xh = F.layer_norm(z, (z.shape[-1],), x["gamma"], x["beta"], eps=B.EPS)
    t = F.linear(xh, x["w_qkvg"]).reshape(n, n, 4, H, C)
    q, k, v, g = t[:, :, 0], t[:, :, 1], t[:, :, 2], t[:, :, 3]     # [i, j, H, c]
    bias = F.linear(xh, x["w_bias"]).permute(2, 0, 1)               # [H, j, k]
    s = torch.einsum("ijhc,ikhc->ihjk", q, k) / C ** 0.5 + bias[None]
    if mask is not None:
        m = mask if not ending else mask.t()
        s = torch.where(m[:, None, None, :].bool(), s, torch.full_like(s, -1e9))
    p = torch.softmax(s, dim=-1)
    a = torch.einsum("ihjk,ikhc->ijhc", p, v)
    o = torch.sigmoid(g) * a
    y = F.linear(o.reshape(n, n, H * C), x["w_o"])
    return y.transpose(0, 1) if ending else y


@pytest.mark.parametrize("ending", [False, True])
def test_block_matches_torch_autograd(ending):
    n = 6
    x = params(n, seed=1)
    mask = inputs.random_mask(n, seed=3, p_keep=0.8)
    leaves = {k: v.clone().requires_grad_(True) for k, v in x.items() if k != "dy"}
    y_t = torch_block({**leaves}, ending, mask)
    (y_t * x["dy"]).sum().backward()
    r = B.block_bwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], x["w_o"], x["dy"], H, C,
                    ending=ending, mask=mask)
    np.testing.assert_allclose(r["y"], y_t.detach().numpy(), rtol=0, atol=1e-11)
    for name, key in [("dz", "z"), ("dgamma", "gamma"), ("dbeta", "beta"), ("dw_qkvg", "w_qkvg"),
                      ("dw_bias", "w_bias"), ("dw_o", "w_o")]:
        ref = leaves[key].grad.numpy()
        err = np.abs(r[name] - ref).max() / np.abs(ref).max()
        assert err < 1e-11, (name, err)


def test_block_finite_differences():
    """Directional central differences of L = sum(y * dy) along random directions, every input."""
    n = 3
    x = params(n, seed=2)
    keys = ["z", "gamma", "beta", "w_qkvg", "w_bias", "w_o"]
    args = {k: x[k].numpy() for k in keys}
    dy = x["dy"].numpy()

    def loss(a):
        return float((B.block_fwd(a["z"], a["gamma"], a["beta"], a["w_qkvg"], a["w_bias"], a["w_o"], H, C)["y"]
                      * dy).sum())

    r = B.block_bwd(args["z"], args["gamma"], args["beta"], args["w_qkvg"], args["w_bias"], args["w_o"], dy, H, C)
    grads = dict(z=r["dz"], gamma=r["dgamma"], beta=r["dbeta"], w_qkvg=r["dw_qkvg"], w_bias=r["dw_bias"],
                 w_o=r["dw_o"])
    rng = np.random.default_rng(0)
    eps = 1e-6
    for key in keys:
        for _ in range(2):
            u = rng.standard_normal(args[key].shape)
            plus = dict(args, **{key: args[key] + eps * u})
            minus = dict(args, **{key: args[key] - eps * u})
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = float((grads[key] * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)


def test_layer_norm_closed_forms():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((4, 5, CZ)) * 3 + 2
    xhat, x_n, mean, rstd = B.layer_norm_fwd(z, np.ones(CZ), np.zeros(CZ))
    np.testing.assert_allclose(xhat.mean(-1), 0, atol=1e-13)
    var = z.var(-1)
    # with gamma = 1, beta = 0: mean of xhat^2 is var / (var + eps) exactly
    np.testing.assert_allclose((xhat ** 2).mean(-1), var / (var + B.EPS), rtol=1e-13)
    np.testing.assert_allclose(mean, z.mean(-1), rtol=1e-14)
    # a pair whose channels are all equal normalises to beta
    zc = np.full((1, 1, CZ), 7.25)
    beta = rng.standard_normal(CZ)
    xc = B.layer_norm_fwd(zc, rng.standard_normal(CZ), beta)[0]
    np.testing.assert_allclose(xc[0, 0], beta, atol=1e-14)
    # same normalisation as torch's layer_norm
    ref = F.layer_norm(torch.from_numpy(z), (CZ,), eps=B.EPS).numpy()
    np.testing.assert_allclose(xhat, ref, atol=1e-12)


def test_projection_layouts_with_identity_weights():
    """Identity weights expose where every projected channel lands in the attention layouts."""
    n = 5
    rng = np.random.default_rng(6)
    z = rng.standard_normal((n, n, CZ))
    gamma, beta = rng.standard_normal(CZ), rng.standard_normal(CZ)
    hc = H * C
    assert hc == CZ
    w = np.concatenate([np.eye(CZ)] * 4, axis=0)            # q = k = v = gate = xhat
    wb = np.eye(CZ)[:H]                                      # bias[h] = xhat channel h
    f = B.ln_proj_fwd(z, gamma, beta, w, wb, H, C)
    xhat = f["xhat"]
    for a in (0, n - 1):
        for b in (0, 2):
            for h in range(H):
                for ch in (0, 5, C - 1):
                    val = xhat[a, b, h * C + ch]
                    assert f["q"][a, h, b, ch] == val and f["k"][a, h, b, ch] == val
                    assert f["v"][a, h, b, ch] == val and f["gate"][a, b, h, ch] == val
                assert f["bias"][h, a, b] == xhat[a, b, h]
    o = rng.standard_normal((n, n, H, C))
    np.testing.assert_array_equal(B.out_proj_fwd(o, np.eye(CZ)), o.reshape(n, n, hc))


def test_projection_backward_is_adjoint():
    """<ln_proj output grads, forward tangent> equals <input grads, input tangent> (dot-product test)."""
    n = 4
    x = params(n, seed=7)
    a = {k: x[k].numpy() for k in ("z", "gamma", "beta", "w_qkvg", "w_bias")}
    rng = np.random.default_rng(8)
    f0 = B.ln_proj_fwd(a["z"], a["gamma"], a["beta"], a["w_qkvg"], a["w_bias"], H, C)
    outs = ("q", "k", "v", "gate", "bias")
    cot = {k: rng.standard_normal(f0[k].shape) for k in outs}
    g = B.ln_proj_bwd(a["z"], a["gamma"], a["beta"], a["w_qkvg"], a["w_bias"], cot["q"], cot["k"], cot["v"],
                      cot["gate"], cot["bias"], H, C)
    tan = {k: rng.standard_normal(a[k].shape) for k in a}
    eps = 1e-6
    fp = B.ln_proj_fwd(*(a[k] + eps * tan[k] for k in ("z", "gamma", "beta", "w_qkvg", "w_bias")), H, C)
    fm = B.ln_proj_fwd(*(a[k] - eps * tan[k] for k in ("z", "gamma", "beta", "w_qkvg", "w_bias")), H, C)
    lhs = sum(float(((fp[k] - fm[k]) / (2 * eps) * cot[k]).sum()) for k in outs)
    rhs = sum(float((g[gk] * tan[k]).sum()) for gk, k in (("dz", "z"), ("dgamma", "gamma"), ("dbeta", "beta"),
                                                          ("dw_qkvg", "w_qkvg"), ("dw_bias", "w_bias")))
    assert abs(lhs - rhs) <= 1e-6 * abs(rhs), (lhs, rhs)


def test_block_ending_is_transpose_conjugate():
    """Block at the ending node == pair transpose of the block at the starting node on transposed z."""
    n = 7
    x = params(n, seed=9)
    a = {k: x[k].numpy() for k in x}
    zt = np.ascontiguousarray(np.transpose(a["z"], (1, 0, 2)))
    dyt = np.ascontiguousarray(np.transpose(a["dy"], (1, 0, 2)))
    end = B.block_bwd(a["z"], a["gamma"], a["beta"], a["w_qkvg"], a["w_bias"], a["w_o"], a["dy"], H, C, ending=True)
    st = B.block_bwd(zt, a["gamma"], a["beta"], a["w_qkvg"], a["w_bias"], a["w_o"], dyt, H, C, ending=False)
    np.testing.assert_allclose(end["y"], np.transpose(st["y"], (1, 0, 2)), atol=1e-12)
    np.testing.assert_allclose(end["dz"], np.transpose(st["dz"], (1, 0, 2)), atol=1e-12)
    for key in ("dgamma", "dbeta", "dw_qkvg", "dw_bias", "dw_o"):
        np.testing.assert_allclose(end[key], st[key], atol=1e-10)
