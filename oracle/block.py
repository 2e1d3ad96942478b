"""fp64 oracle for the pair-representation block around the triangle attention.

TEST INFRASTRUCTURE ONLY (the same rule as the rest of this package: only
``tests/``, the smoke check and the benchmark's CPU baseline call it).

The block (TurboPairFormer news item, "Dove si impiega il tempo": the pair
stack spends its time in the triangle attention and in the LayerNorm and
linear layers around it; ScaleFold summary, core contributions: fused
LayerNorm / linear kernels; HelixFold review, "Fused Gated Self-Attention"):

    x_n   = (z - mean(z)) / sqrt(var(z) + eps)          per pair, biased variance
    xhat  = x_n * gamma + beta
    q|k|v|g = xhat @ w_qkvg.T   split into 4 blocks of H*c, each [pair, h, c]
    b       = xhat @ w_bias.T   [pair, h]
    o       = triangle attention (starting or ending node) of q, k, v, b, g
    y       = o_flat @ w_o.T    o_flat [pair, h*c]

Layouts (pair = (a, b), a the first pair axis):
    z, y            [N, N, cz]
    w_qkvg          [4*H*c, cz]   rows: q (h*c + ch), then k, v, gate
    w_bias          [H, cz]
    w_o             [cz_out, H*c]
    q, k, v         [a, H, b, c]      gate, o  [a, b, H, c]      bias [H, a, b]
Weights follow the (out, in) convention of a linear layer; there are no
linear biases.  The LayerNorm, the projections and the output linear act on
each pair alone, so the ending node of the block is the block's starting node
conjugated by the pair transpose; only the attention call differs.

Every step is a plain numpy float64 expression (matmul / sum as library
primitives), in the order written above, with no fusion or blocking.
"""
from __future__ import annotations

import numpy as np

from . import _f64, attn_bwd, attn_end_bwd, attn_end_fwd, attn_fwd

EPS = 1e-5


def layer_norm_fwd(z, gamma, beta, eps: float = EPS):
    """Per-pair LayerNorm over the last axis.  Returns (xhat, x_n, mean, rstd)."""
    z = _f64(z)
    mean = z.mean(axis=-1)
    var = ((z - mean[..., None]) ** 2).mean(axis=-1)
    rstd = 1.0 / np.sqrt(var + eps)
    x_n = (z - mean[..., None]) * rstd[..., None]
    xhat = x_n * _f64(gamma) + _f64(beta)
    return xhat, x_n, mean, rstd


def layer_norm_bwd(dxhat, x_n, rstd, gamma):
    """Gradients of the LayerNorm: returns (dz, dgamma, dbeta) summed over pairs."""
    cz = x_n.shape[-1]
    dgamma = (dxhat * x_n).reshape(-1, cz).sum(axis=0)
    dbeta = dxhat.reshape(-1, cz).sum(axis=0)
    g = dxhat * _f64(gamma)
    dz = rstd[..., None] * (g - g.mean(axis=-1, keepdims=True) - x_n * (g * x_n).mean(axis=-1, keepdims=True))
    return dz, dgamma, dbeta


def ln_proj_fwd(z, gamma, beta, w_qkvg, w_bias, h: int, c: int, eps: float = EPS):
    """LayerNorm + the five projections; outputs in the attention's layouts."""
    xhat, x_n, mean, rstd = layer_norm_fwd(z, gamma, beta, eps)
    n0, n1, _ = xhat.shape
    t = xhat @ _f64(w_qkvg).T                     # [a, b, 4*H*c]
    t = t.reshape(n0, n1, 4, h, c)
    q, k, v = (np.ascontiguousarray(np.transpose(t[:, :, s], (0, 2, 1, 3))) for s in range(3))
    gate = np.ascontiguousarray(t[:, :, 3])        # [a, b, H, c]
    bias = np.ascontiguousarray(np.transpose(xhat @ _f64(w_bias).T, (2, 0, 1)))  # [H, a, b]
    return dict(q=q, k=k, v=v, gate=gate, bias=bias, mean=mean, rstd=rstd, xhat=xhat, x_n=x_n)


def ln_proj_bwd(z, gamma, beta, w_qkvg, w_bias, dq, dk, dv, dgate, dbias, h: int, c: int, eps: float = EPS):
    """Backward of ln_proj_fwd given the gradients of its five outputs."""
    xhat, x_n, mean, rstd = layer_norm_fwd(z, gamma, beta, eps)
    n0, n1, cz = xhat.shape
    dq, dk, dv, dgate, dbias = (_f64(t) for t in (dq, dk, dv, dgate, dbias))
    # gradient of the concatenated projection output, [a, b, 4, H, c]
    dt = np.stack([np.transpose(dq, (0, 2, 1, 3)), np.transpose(dk, (0, 2, 1, 3)),
                   np.transpose(dv, (0, 2, 1, 3)), dgate], axis=2).reshape(n0, n1, 4 * h * c)
    db = np.transpose(dbias, (1, 2, 0))            # [a, b, H]
    dxhat = dt @ _f64(w_qkvg) + db @ _f64(w_bias)
    dw_qkvg = dt.reshape(-1, 4 * h * c).T @ xhat.reshape(-1, cz)
    dw_bias = db.reshape(-1, h).T @ xhat.reshape(-1, cz)
    dz, dgamma, dbeta = layer_norm_bwd(dxhat, x_n, rstd, gamma)
    return dict(dz=dz, dgamma=dgamma, dbeta=dbeta, dw_qkvg=dw_qkvg, dw_bias=dw_bias, dxhat=dxhat)


def out_proj_fwd(o, w_o):
    """y[a, b, :] = o[a, b, :, :].flatten() @ w_o.T."""
    o = _f64(o)
    n0, n1 = o.shape[:2]
    return o.reshape(n0, n1, -1) @ _f64(w_o).T


def out_proj_bwd(o, w_o, dy):
    o, dy = _f64(o), _f64(dy)
    n0, n1 = o.shape[:2]
    of = o.reshape(n0 * n1, -1)
    d_o = (dy.reshape(n0 * n1, -1) @ _f64(w_o)).reshape(o.shape)
    dw_o = dy.reshape(n0 * n1, -1).T @ of
    return dict(do=d_o, dw_o=dw_o)


def block_fwd(z, gamma, beta, w_qkvg, w_bias, w_o, h: int, c: int, ending: bool = False, mask=None,
              eps: float = EPS):
    """Whole block forward: LayerNorm + projections -> attention -> output linear."""
    f = ln_proj_fwd(z, gamma, beta, w_qkvg, w_bias, h, c, eps)
    att = (attn_end_fwd if ending else attn_fwd)(f["q"], f["k"], f["v"], f["bias"], f["gate"], mask)
    y = out_proj_fwd(att["out"], w_o)
    return dict(y=y, front=f, attn=att)


def block_bwd(z, gamma, beta, w_qkvg, w_bias, w_o, dy, h: int, c: int, ending: bool = False, mask=None,
              eps: float = EPS):
    """Whole block forward + backward.  Returns y and every input / weight gradient."""
    f = ln_proj_fwd(z, gamma, beta, w_qkvg, w_bias, h, c, eps)
    fwd = attn_end_fwd if ending else attn_fwd
    att = fwd(f["q"], f["k"], f["v"], f["bias"], f["gate"], mask)
    y = out_proj_fwd(att["out"], w_o)
    ob = out_proj_bwd(att["out"], w_o, dy)
    bwd = attn_end_bwd if ending else attn_bwd
    ab = bwd(f["q"], f["k"], f["v"], f["bias"], f["gate"], mask, ob["do"])
    fb = ln_proj_bwd(z, gamma, beta, w_qkvg, w_bias, ab["dq"], ab["dk"], ab["dv"], ab["dgate"], ab["dbias"],
                     h, c, eps)
    return dict(y=y, out=att["out"], dz=fb["dz"], dgamma=fb["dgamma"], dbeta=fb["dbeta"],
                dw_qkvg=fb["dw_qkvg"], dw_bias=fb["dw_bias"], dw_o=ob["dw_o"], front=f, attn_grads=ab,
                do=ob["do"])
