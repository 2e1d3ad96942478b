"""Pins of the fp64 oracle to things other than itself (CPU only).

Each check ties the oracle to a library routine, a closed form, an invariant,
finite differences or a brute-force evaluation, chosen so that a plausible
slip (transposed bias, wrong scale, wrong gate layout, dropped term in the
softmax backward, sign error, wrong mask handling) fails at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit

import oracle

RNG = np.random.default_rng(12345)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def make(rows, H, N, c, nk=None, bias_scale=1.0):
    nk = N if nk is None else nk
    return dict(q=rand(rows, H, N, c), k=rand(rows, H, nk, c), v=rand(rows, H, nk, c),
                bias=rand(H, N, nk, scale=bias_scale), gate=rand(rows, N, H, c), dout=rand(rows, N, H, c))


# --------------------------------------------------------------------------- forward

def brute_forward(q, k, v, bias, gate, mask):
    """Element-by-element evaluation with Python loops and math.exp."""
    rows, H, N, c = q.shape
    nk = k.shape[2]
    out = np.zeros((rows, N, H, c))
    lse = np.zeros((rows, H, N))
    for i in range(rows):
        for h in range(H):
            for j in range(N):
                logits = []
                for kk in range(nk):
                    if mask is not None and mask[i, kk] == 0:
                        logits.append(-1e9)
                        continue
                    d = 0.0
                    for x in range(c):
                        d += q[i, h, j, x] * k[i, h, kk, x]
                    logits.append(d / math.sqrt(c) + bias[h, j, kk])
                m = max(logits)
                ex = [math.exp(s - m) for s in logits]
                tot = sum(ex)
                lse[i, h, j] = m + math.log(tot)
                for x in range(c):
                    a = sum(ex[kk] / tot * v[i, h, kk, x] for kk in range(nk))
                    out[i, j, h, x] = a / (1.0 + math.exp(-gate[i, j, h, x]))
    return out, lse


@pytest.mark.parametrize("N", [1, 2, 3, 4, 7])
def test_brute_force_small(N):
    x = make(N, 2, N, 5)
    mask = None
    if N >= 3:
        mask = (RNG.random((N, N)) < 0.7).astype(np.uint8)
        mask[:, 0] = 1
    r = oracle.attn_fwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], mask, threads=1)
    out, lse = brute_forward(x["q"], x["k"], x["v"], x["bias"], x["gate"], mask)
    np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-12, atol=1e-13)


def _sdpa(q, k, v, bias, mask):
    """torch scaled_dot_product_attention (float64, CPU) with the pair bias as additive mask."""
    Q, K, V = (torch.from_numpy(t) for t in (q, k, v))
    am = torch.from_numpy(bias)[None].expand(q.shape[0], -1, -1, -1).clone()
    if mask is not None:
        add = torch.where(torch.from_numpy(mask != 0), 0.0, float("-inf")).to(torch.float64)
        am = am + add[:, None, None, :]
    return F.scaled_dot_product_attention(Q, K, V, attn_mask=am, scale=1.0 / math.sqrt(q.shape[-1])).numpy()


@pytest.mark.parametrize("with_mask", [False, True])
def test_sdpa_special_case(with_mask):
    """gate = +40 makes sigmoid == 1 in fp64: the output is plain biased attention."""
    rows, H, N, c = 5, 4, 9, 32
    x = make(rows, H, N, c, bias_scale=2.0)
    gate = np.full((rows, N, H, c), 40.0)
    mask = None
    if with_mask:
        mask = (RNG.random((rows, N)) < 0.6).astype(np.uint8)
        mask[:, 3] = 1
    r = oracle.attn_fwd(x["q"], x["k"], x["v"], x["bias"], gate, mask)
    ref = _sdpa(x["q"], x["k"], x["v"], x["bias"], mask)
    np.testing.assert_allclose(r["attn"], ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["out"], np.transpose(ref, (0, 2, 1, 3)), rtol=1e-11, atol=1e-12)


def test_lse_and_gate_layout():
    """lse against torch.logsumexp of library-computed logits; out = expit(gate) * attn in pair layout."""
    rows, H, N, c = 3, 4, 11, 32
    x = make(rows, H, N, c)
    r = oracle.attn_fwd(x["q"], x["k"], x["v"], x["bias"], x["gate"])
    logits = torch.matmul(torch.from_numpy(x["q"]), torch.from_numpy(x["k"]).transpose(-1, -2)) / math.sqrt(c)
    logits = logits + torch.from_numpy(x["bias"])[None]
    np.testing.assert_allclose(r["lse"], torch.logsumexp(logits, dim=-1).numpy(), rtol=1e-12, atol=1e-12)
    gated = expit(x["gate"]) * np.transpose(r["attn"], (0, 2, 1, 3))
    np.testing.assert_allclose(r["out"], gated, rtol=1e-12, atol=1e-13)


def test_closed_forms():
    H, c = 3, 32
    # N = 1: the only key gets weight 1
    x = make(1, H, 1, c)
    r = oracle.attn_fwd(x["q"], x["k"], x["v"], x["bias"], x["gate"])
    np.testing.assert_allclose(r["attn"], x["v"], rtol=1e-14, atol=0)
    # constant values: softmax rows sum to one
    rows, N = 4, 13
    x = make(rows, H, N, c)
    u = rand(c)
    v = np.broadcast_to(u, (rows, H, N, c)).copy()
    r = oracle.attn_fwd(x["q"], x["k"], v, x["bias"], x["gate"])
    np.testing.assert_allclose(r["attn"], np.broadcast_to(u, r["attn"].shape), rtol=1e-13, atol=1e-13)
    # q = 0, bias = 0: uniform weights, a = mean of v over keys
    r = oracle.attn_fwd(np.zeros_like(x["q"]), x["k"], x["v"], np.zeros_like(x["bias"]), x["gate"])
    np.testing.assert_allclose(r["attn"], np.broadcast_to(x["v"].mean(axis=2, keepdims=True), r["attn"].shape),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r["lse"], np.full(r["lse"].shape, math.log(N)), rtol=1e-14)
    # bias -1e9 everywhere except key kstar: a = v[kstar]
    kstar = 5
    b = np.full((H, N, N), -1e9)
    b[:, :, kstar] = 0.0
    r = oracle.attn_fwd(x["q"], x["k"], x["v"], b, x["gate"])
    np.testing.assert_allclose(r["attn"], np.broadcast_to(x["v"][:, :, kstar:kstar + 1, :], r["attn"].shape),
                               rtol=1e-13, atol=1e-13)


def test_bias_shift_invariance():
    rows, H, N, c = 3, 4, 10, 32
    x = make(rows, H, N, c)
    shift = rand(H, N, 1) * 3.0
    r0 = oracle.attn_fwd(x["q"], x["k"], x["v"], x["bias"], x["gate"])
    r1 = oracle.attn_fwd(x["q"], x["k"], x["v"], x["bias"] + shift, x["gate"])
    np.testing.assert_allclose(r1["out"], r0["out"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r1["lse"], r0["lse"] + shift[None, :, :, 0], rtol=1e-12, atol=1e-12)


def test_query_subset_is_exact():
    """Evaluating a subset of queries (all keys) reproduces those rows of the full result."""
    rows, H, N, c = 4, 2, 12, 32
    x = make(rows, H, N, c)
    full = oracle.attn_bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], None, x["dout"])
    sel = np.array([0, 5, 11])
    sub = oracle.attn_bwd(x["q"][:, :, sel], x["k"], x["v"], x["bias"][:, sel], x["gate"][:, sel], None,
                          x["dout"][:, sel])
    np.testing.assert_allclose(sub["out"], full["out"][:, sel], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sub["dq"], full["dq"][:, :, sel], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sub["dbias"], full["dbias"][:, sel], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sub["dgate"], full["dgate"][:, sel], rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- backward

def _loss(x, mask):
    r = oracle.attn_fwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], mask, threads=1)
    return float(np.sum(r["out"] * x["dout"]))


@pytest.mark.parametrize("N,with_mask", [(2, False), (3, False), (4, True)])
def test_finite_differences(N, with_mask):
    """Central differences (step 1e-6, fp64) of L = sum(out * dout) on sampled elements, H=4, c=32."""
    H, c = 4, 32
    x = make(N, H, N, c)
    mask = None
    if with_mask:
        mask = np.ones((N, N), dtype=np.uint8)
        mask[0, 1] = 0
        mask[2, 3] = 0
    r = oracle.attn_bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], mask, x["dout"], threads=1)
    grads = dict(q=r["dq"], k=r["dk"], v=r["dv"], bias=r["dbias"], gate=r["dgate"])
    step = 1e-6
    rng = np.random.default_rng(N)
    for name, gref in grads.items():
        flat = x[name].reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 40), replace=False)
        for e in idx:
            orig = flat[e]
            flat[e] = orig + step
            lp = _loss(x, mask)
            flat[e] = orig - step
            lm = _loss(x, mask)
            flat[e] = orig
            fd = (lp - lm) / (2 * step)
            an = gref.reshape(-1)[e]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}[{e}]: fd {fd} vs analytic {an}"


def _torch_autograd(x, mask):
    """Gradients of the composed expression by torch autograd (float64 CPU)."""
    t = {k: torch.from_numpy(v.copy()).requires_grad_(k != "dout") for k, v in x.items()}
    c = t["q"].shape[-1]
    logits = torch.matmul(t["q"], t["k"].transpose(-1, -2)) / math.sqrt(c) + t["bias"][None]
    if mask is not None:
        keep = torch.from_numpy(mask != 0)[:, None, None, :]
        logits = torch.where(keep, logits, torch.full_like(logits, -1e9))
    p = torch.softmax(logits, dim=-1)
    a = torch.matmul(p, t["v"])
    out = torch.sigmoid(t["gate"]) * a.permute(0, 2, 1, 3)
    (out * t["dout"]).sum().backward()
    return {k: t[k].grad.numpy() for k in ("q", "k", "v", "bias", "gate")}, out.detach().numpy()


@pytest.mark.parametrize("N,with_mask", [(16, False), (24, True)])
def test_torch_autograd(N, with_mask):
    H, c = 4, 32
    x = make(N, H, N, c, bias_scale=2.0)
    mask = None
    if with_mask:
        mask = (RNG.random((N, N)) < 0.75).astype(np.uint8)
        mask[:, 2] = 1
    r = oracle.attn_bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], mask, x["dout"])
    g, out = _torch_autograd(x, mask)
    np.testing.assert_allclose(r["out"], out, rtol=1e-11, atol=1e-13)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("bias", "dbias"), ("gate", "dgate")):
        np.testing.assert_allclose(r[key], g[name], rtol=1e-10, atol=1e-12, err_msg=name)


def test_backward_invariants():
    rows, H, N, c = 6, 4, 14, 32
    x = make(rows, H, N, c)
    r = oracle.attn_bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], None, x["dout"])
    # the two forms of D agree
    assert r["d_mismatch"] < 1e-12
    # softmax gradient rows sum to zero -> dbias rows sum to zero
    np.testing.assert_allclose(r["dbias"].sum(axis=-1), 0.0, atol=1e-12)
    # sum_k dv = sum_j dA, dA = dout * sigmoid(gate) in kernel order
    dA = np.transpose(x["dout"] * expit(x["gate"]), (0, 2, 1, 3))
    np.testing.assert_allclose(r["dv"].sum(axis=2), dA.sum(axis=2), rtol=1e-11, atol=1e-12)
    # shifting every key of a row by the same vector leaves the softmax (and dq) unchanged
    u = rand(rows, H, 1, c)
    r2 = oracle.attn_bwd(x["q"], x["k"] + u, x["v"], x["bias"], x["gate"], None, x["dout"])
    np.testing.assert_allclose(r2["dq"], r["dq"], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r2["out"], r["out"], rtol=1e-11, atol=1e-13)
    # gradients are linear in dout
    r3 = oracle.attn_bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], None, 2.5 * x["dout"])
    for key in ("dq", "dk", "dv", "dbias", "dgate"):
        np.testing.assert_allclose(r3[key], 2.5 * r[key], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- mask

def test_mask_semantics():
    rows, H, N, c = 5, 4, 12, 32
    x = make(rows, H, N, c)
    mask = (RNG.random((rows, N)) < 0.6).astype(np.uint8)
    mask[:, 0] = 1
    mask[:, 7] = 0           # key 7 masked in every row
    mask[3, :] = 0           # row 3: every key masked
    r = oracle.attn_bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], mask, x["dout"])
    for i in range(rows):
        dead = mask[i] == 0
        if i != 3:
            assert np.all(r["dk"][i][:, dead] == 0.0)
            assert np.all(r["dv"][i][:, dead] == 0.0)
    assert np.all(r["dbias"][:, :, 7] == 0.0)
    # fully masked row: uniform weights, no gradient into q, k or bias
    np.testing.assert_allclose(r["attn"][3], np.broadcast_to(x["v"][3].mean(axis=1, keepdims=True), (H, N, c)),
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["lse"][3], -1e9 + math.log(N), rtol=1e-15)
    assert np.all(r["dq"][3] == 0.0) and np.all(r["dk"][3] == 0.0)
    dA3 = np.transpose(x["dout"][3] * expit(x["gate"][3]), (1, 0, 2))  # [H,N,c]
    np.testing.assert_allclose(r["dv"][3], np.broadcast_to(dA3.mean(axis=1, keepdims=True), (H, N, c)),
                               rtol=1e-12, atol=1e-13)
    # randomising k, v, bias at masked keys changes nothing
    k2, v2, b2 = x["k"].copy(), x["v"].copy(), x["bias"].copy()
    for i in range(rows):
        if i == 3:
            continue
        dead = mask[i] == 0
        k2[i][:, dead] = rand(H, int(dead.sum()), c)
        v2[i][:, dead] = rand(H, int(dead.sum()), c)
    b2[:, :, 7] = rand(H, N)
    r2 = oracle.attn_bwd(x["q"], k2, v2, b2, x["gate"], mask, x["dout"])
    keep_rows = [i for i in range(rows) if i != 3]
    np.testing.assert_array_equal(r2["out"][keep_rows], r["out"][keep_rows])
    np.testing.assert_array_equal(r2["dq"][keep_rows], r["dq"][keep_rows])


# --------------------------------------------------------------------------- ending node

def direct_end_forward(q, k, v, bias, gate):
    """Ending node written with explicit indices: o_ij = sig(g_ij) sum_k softmax_k(q_ij.k_kj/sqrt(c) + b_ki) v_kj.

    Tensors are in the pair layout: q[a,h,b,:] is the query of pair (a, b);
    gate[a,b,h,:]; bias[h,x,y] is the bias of pair (x, y).
    """
    N, H, _, c = q.shape
    logits = np.einsum("ihjc,khjc->jhik", q, k) / math.sqrt(c)   # [j,h,i,k] : q_ij . k_kj
    logits = logits + np.transpose(bias, (0, 2, 1))[None]         # b_ki -> bias[h,k,i] at [.,h,i,k]
    logits -= logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=-1, keepdims=True)
    a = np.einsum("jhik,khjc->ijhc", p, v)                        # [i,j,h,c]
    return expit(gate) * a


def test_ending_node_identity():
    N, H, c = 9, 4, 32
    x = make(N, H, N, c, bias_scale=2.0)
    r = oracle.attn_end_fwd(x["q"], x["k"], x["v"], x["bias"], x["gate"])
    np.testing.assert_allclose(r["out"], direct_end_forward(x["q"], x["k"], x["v"], x["bias"], x["gate"]),
                               rtol=1e-12, atol=1e-13)


def test_ending_node_gradients_fd():
    N, H, c = 3, 2, 32
    x = make(N, H, N, c)
    r = oracle.attn_end_bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], None, x["dout"])

    def loss():
        return float(np.sum(direct_end_forward(x["q"], x["k"], x["v"], x["bias"], x["gate"]) * x["dout"]))

    rng = np.random.default_rng(7)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("bias", "dbias"), ("gate", "dgate")):
        flat = x[name].reshape(-1)
        for e in rng.choice(flat.size, size=15, replace=False):
            o = flat[e]
            flat[e] = o + 1e-6
            lp = loss()
            flat[e] = o - 1e-6
            lm = loss()
            flat[e] = o
            fd = (lp - lm) / 2e-6
            an = r[key].reshape(-1)[e]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}[{e}]"
