"""fp64 oracle of the triangular multiplicative update (outgoing and incoming edges).

TEST INFRASTRUCTURE ONLY: only ``tests/``, the smoke check and the benchmark's
CPU baseline call it.  It shares no code with the GPU library and never
imports it.

What the pages say.  The TurboPairFormer news item ("Dove si impiega il tempo",
"Benchmark di addestramento") names triangle multiplication as the other
operation of the pair stack that its kernels implement next to triangle
attention, and integrates its own triangle-multiplication kernels into
OpenFold3.  No page writes the operation out.  The reading taken is the
triangular multiplicative update of the AlphaFold family as OpenFold3's
Pairformer uses it (linear layers without biases, as in this package's
attention block), written here from its published definition:

    x      = LayerNorm(z)                         per pair over c_z, gamma_in / beta_in
    a      = sigmoid(x W_ag^T) * (x W_ap^T)       [N, N, c]
    b      = sigmoid(x W_bg^T) * (x W_bp^T)       [N, N, c]
    g      = sigmoid(x W_g^T)                     [N, N, c_z]
    t_ij   = sum_k a_ik * b_jk       (outgoing edges)
    t_ij   = sum_k a_ki * b_kj       (incoming edges)
    y      = g * (LayerNorm(t) W_o^T)             LayerNorm over c, gamma_out / beta_out

Weights use the (out, in) convention of a linear layer: w_in [4c + c_z, c_z]
holds the rows of W_ap, W_ag, W_bp, W_bg (c rows each) and W_g (c_z rows), in
that order; w_out [c_z, c].  LayerNorms use the biased variance and eps = 1e-5.
Every step is a plain numpy float64 expression in the order written above
(matmul and sum as library primitives; the contraction over the third token is
one matrix product per channel), with no blocking or fusion.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-5


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def layer_norm(x, gamma, beta, eps=EPS):
    """Returns (y, x_n, rstd) over the last axis."""
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    x_n = (x - mean) * rstd
    return x_n * gamma + beta, x_n, rstd


def layer_norm_bwd(dy, x_n, rstd, gamma):
    """Gradient of y = x_n * gamma + beta with respect to x, gamma and beta (sums over every leading axis)."""
    width = x_n.shape[-1]
    g = dy * gamma
    dx = rstd * (g - g.mean(axis=-1, keepdims=True) - x_n * (g * x_n).mean(axis=-1, keepdims=True))
    return dx, (dy * x_n).reshape(-1, width).sum(axis=0), dy.reshape(-1, width).sum(axis=0)


def split_w_in(w_in, c):
    """Rows of w_in: W_ap, W_ag, W_bp, W_bg (c each), then W_g."""
    return w_in[:c], w_in[c:2 * c], w_in[2 * c:3 * c], w_in[3 * c:4 * c], w_in[4 * c:]


def _cf(x):
    """[n, n, c] -> channel-first [c, n, n] copy (x_cf[c, r, s] = x[r, s, c])."""
    return np.ascontiguousarray(np.transpose(x, (2, 0, 1)))


def _pl(x):
    """channel-first [c, n, n] -> [n, n, c]."""
    return np.ascontiguousarray(np.transpose(x, (1, 2, 0)))


def contract(a, b, incoming):
    """t_ij = sum_k a_ik b_jk (outgoing) or sum_k a_ki b_kj (incoming), per channel, as one matrix product per
    channel: T_c = A_c B_c^T, or A_c^T B_c for incoming edges (A_c[r, s] = a[r, s, c])."""
    ac, bc = _cf(a), _cf(b)
    if incoming:
        return _pl(np.matmul(np.transpose(ac, (0, 2, 1)), bc))
    return _pl(np.matmul(ac, np.transpose(bc, (0, 2, 1))))


def trimul_fwd(z, gamma_in, beta_in, w_in, gamma_out, beta_out, w_out, incoming=False, eps=EPS):
    """Forward.  z [N, N, c_z].  Returns a dict with y and every intermediate."""
    z, gamma_in, beta_in, w_in, gamma_out, beta_out, w_out = (
        _f64(t) for t in (z, gamma_in, beta_in, w_in, gamma_out, beta_out, w_out))
    c = w_out.shape[1]
    w_ap, w_ag, w_bp, w_bg, w_g = split_w_in(w_in, c)
    x, x_n, rstd_in = layer_norm(z, gamma_in, beta_in, eps)
    ap, ag, bp, bg, gp = x @ w_ap.T, x @ w_ag.T, x @ w_bp.T, x @ w_bg.T, x @ w_g.T
    a = sigmoid(ag) * ap
    b = sigmoid(bg) * bp
    g = sigmoid(gp)
    t = contract(a, b, incoming)
    tl, t_n, rstd_out = layer_norm(t, gamma_out, beta_out, eps)
    u = tl @ w_out.T
    y = g * u
    return dict(y=y, x=x, x_n=x_n, rstd_in=rstd_in, ap=ap, ag=ag, bp=bp, bg=bg, gp=gp, a=a, b=b, g=g, t=t,
                tl=tl, t_n=t_n, rstd_out=rstd_out, u=u)


def trimul_bwd(z, gamma_in, beta_in, w_in, gamma_out, beta_out, w_out, dy, incoming=False, eps=EPS):
    """Forward and backward.  Returns y, the gradients of z and of every parameter, and the gradients of the
    intermediates (da, db, dt) the kernels produce on the way."""
    f = trimul_fwd(z, gamma_in, beta_in, w_in, gamma_out, beta_out, w_out, incoming, eps)
    w_in, gamma_in, gamma_out, w_out, dy = (_f64(t) for t in (w_in, gamma_in, gamma_out, w_out, dy))
    c = w_out.shape[1]
    cz = w_out.shape[0]
    w_ap, w_ag, w_bp, w_bg, w_g = split_w_in(w_in, c)
    # y = g * u
    dg = dy * f["u"]
    du = dy * f["g"]
    # u = tl w_out^T
    dw_out = du.reshape(-1, cz).T @ f["tl"].reshape(-1, c)
    dtl = du @ w_out
    dt, dgamma_out, dbeta_out = layer_norm_bwd(dtl, f["t_n"], f["rstd_out"], gamma_out)
    # t = contract(a, b), per channel: outgoing T = A B^T gives dA = dT B, dB = dT^T A;
    # incoming T = A^T B gives dA = B dT^T, dB = A dT
    ac, bc, dtc = _cf(f["a"]), _cf(f["b"]), _cf(dt)
    if incoming:
        da = _pl(np.matmul(bc, np.transpose(dtc, (0, 2, 1))))
        db = _pl(np.matmul(ac, dtc))
    else:
        da = _pl(np.matmul(dtc, bc))
        db = _pl(np.matmul(np.transpose(dtc, (0, 2, 1)), ac))
    # gates: a = s(ag) ap, b = s(bg) bp, g = s(gp)
    sa, sb = sigmoid(f["ag"]), sigmoid(f["bg"])
    dap = da * sa
    dag = da * f["ap"] * sa * (1.0 - sa)
    dbp = db * sb
    dbg = db * f["bp"] * sb * (1.0 - sb)
    dgp = dg * f["g"] * (1.0 - f["g"])
    dpre = np.concatenate([dap, dag, dbp, dbg, dgp], axis=-1)          # [N, N, 4c + c_z]
    w_all = np.concatenate([w_ap, w_ag, w_bp, w_bg, w_g], axis=0)
    dx = dpre @ w_all
    dw_in = dpre.reshape(-1, w_all.shape[0]).T @ f["x"].reshape(-1, cz)
    dz, dgamma_in, dbeta_in = layer_norm_bwd(dx, f["x_n"], f["rstd_in"], gamma_in)
    return dict(y=f["y"], dz=dz, dgamma_in=dgamma_in, dbeta_in=dbeta_in, dw_in=dw_in, dgamma_out=dgamma_out,
                dbeta_out=dbeta_out, dw_out=dw_out, da=da, db=db, dt=dt, dg=dg, fwd=f)
