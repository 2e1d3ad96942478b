"""Pins of the triangular multiplicative update oracle (oracle/trimul.py), on the CPU.

Each pin is fixed by something other than the oracle's own expressions:
* literal per-element loops over (i, j, k, channel) in pure Python scalars at
  tiny sizes, both edge directions;
* torch float64 autograd of the composition written with torch's own
  layer_norm / linear / sigmoid / einsum, for the output and every gradient;
* central finite differences of <y, dy> along random directions;
* the identity incoming(z; W_a, W_b) = T(outgoing(T(z); W_b, W_a)), where T
  swaps the two pair axes (which a wrong contraction index breaks);
* closed forms: W_ap = 0 gives t = 0, so y = g * (beta_out W_o^T); N = 1 gives
  t = a * b.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import trimul as TM


def params(n, cz, c, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, n, cz))
    w_in = rng.standard_normal((4 * c + cz, cz)) / math.sqrt(cz) * scale
    w_out = rng.standard_normal((cz, c)) / math.sqrt(c)
    gi, bi = 1.0 + 0.1 * rng.standard_normal(cz), 0.1 * rng.standard_normal(cz)
    go, bo = 1.0 + 0.1 * rng.standard_normal(c), 0.1 * rng.standard_normal(c)
    dy = rng.standard_normal((n, n, cz))
    return dict(z=z, gamma_in=gi, beta_in=bi, w_in=w_in, gamma_out=go, beta_out=bo, w_out=w_out), dy


def brute_force_y(p, incoming):
    """y by explicit loops over pairs, channels and the third token (plain Python floats)."""
    z, w_in, w_out = p["z"], p["w_in"], p["w_out"]
    n, _, cz = z.shape
    c = w_out.shape[1]
    eps = 1e-5

    def ln(vec, gam, bet):
        m = sum(vec) / len(vec)
        var = sum((v - m) ** 2 for v in vec) / len(vec)
        r = 1.0 / math.sqrt(var + eps)
        return [(v - m) * r * gam[q] + bet[q] for q, v in enumerate(vec)]

    def sig(v):
        return 1.0 / (1.0 + math.exp(-v))

    def lin(row, w, o):
        return sum(w[o][q] * row[q] for q in range(len(row)))

    a = [[None] * n for _ in range(n)]
    b = [[None] * n for _ in range(n)]
    g = [[None] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            x = ln(list(z[i][j]), p["gamma_in"], p["beta_in"])
            a[i][j] = [sig(lin(x, w_in, c + q)) * lin(x, w_in, q) for q in range(c)]
            b[i][j] = [sig(lin(x, w_in, 3 * c + q)) * lin(x, w_in, 2 * c + q) for q in range(c)]
            g[i][j] = [sig(lin(x, w_in, 4 * c + o)) for o in range(cz)]
    y = np.zeros((n, n, cz))
    for i in range(n):
        for j in range(n):
            t = []
            for q in range(c):
                s = 0.0
                for k in range(n):
                    s += a[k][i][q] * b[k][j][q] if incoming else a[i][k][q] * b[j][k][q]
                t.append(s)
            tl = ln(t, p["gamma_out"], p["beta_out"])
            for o in range(cz):
                y[i][j][o] = g[i][j][o] * lin(tl, w_out, o)
    return y


@pytest.mark.parametrize("incoming", [False, True])
def test_brute_force(incoming):
    p, _ = params(3, 4, 5, seed=1)
    ref = brute_force_y(p, incoming)
    got = TM.trimul_fwd(**p, incoming=incoming)["y"]
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def torch_composition(p, dy, incoming):
    """The update written with torch primitives; autograd gives every gradient."""
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    c = p["w_out"].shape[1]
    cz = p["z"].shape[-1]
    x = torch.nn.functional.layer_norm(t["z"], (cz,), t["gamma_in"], t["beta_in"], eps=1e-5)
    w_ap, w_ag, w_bp, w_bg, w_g = torch.split(t["w_in"], [c, c, c, c, cz], dim=0)
    lin = torch.nn.functional.linear
    a = torch.sigmoid(lin(x, w_ag)) * lin(x, w_ap)
    b = torch.sigmoid(lin(x, w_bg)) * lin(x, w_bp)
    g = torch.sigmoid(lin(x, w_g))
    tt = torch.einsum("kic,kjc->ijc", a, b) if incoming else torch.einsum("ikc,jkc->ijc", a, b)
    y = g * lin(torch.nn.functional.layer_norm(tt, (c,), t["gamma_out"], t["beta_out"], eps=1e-5), t["w_out"])
    (y * torch.tensor(dy)).sum().backward()
    return y.detach().numpy(), {k: v.grad.numpy() for k, v in t.items()}


@pytest.mark.parametrize("incoming", [False, True])
@pytest.mark.parametrize("n,cz,c", [(5, 8, 6), (4, 128, 128)])
def test_torch_autograd(incoming, n, cz, c):
    p, dy = params(n, cz, c, seed=2 + n)
    y_ref, g_ref = torch_composition(p, dy, incoming)
    r = TM.trimul_bwd(**p, dy=dy, incoming=incoming)
    assert np.allclose(r["y"], y_ref, rtol=1e-11, atol=1e-11)
    names = dict(z="dz", gamma_in="dgamma_in", beta_in="dbeta_in", w_in="dw_in", gamma_out="dgamma_out",
                 beta_out="dbeta_out", w_out="dw_out")
    for k, name in names.items():
        scale = max(1.0, np.max(np.abs(g_ref[k])))
        assert np.max(np.abs(r[name] - g_ref[k])) <= 1e-10 * scale, name


@pytest.mark.parametrize("incoming", [False, True])
def test_finite_differences(incoming):
    p, dy = params(3, 6, 5, seed=7)
    r = TM.trimul_bwd(**p, dy=dy, incoming=incoming)
    rng = np.random.default_rng(8)
    names = dict(z="dz", gamma_in="dgamma_in", beta_in="dbeta_in", w_in="dw_in", gamma_out="dgamma_out",
                 beta_out="dbeta_out", w_out="dw_out")
    h = 1e-6
    for k, name in names.items():
        d = rng.standard_normal(p[k].shape)
        pp, pm = dict(p), dict(p)
        pp[k] = p[k] + h * d
        pm[k] = p[k] - h * d
        fd = (np.sum(TM.trimul_fwd(**pp, incoming=incoming)["y"] * dy) -
              np.sum(TM.trimul_fwd(**pm, incoming=incoming)["y"] * dy)) / (2 * h)
        an = float(np.sum(r[name] * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_incoming_is_transposed_outgoing_with_swapped_operands():
    p, dy = params(5, 8, 6, seed=11)
    c = p["w_out"].shape[1]
    w = p["w_in"]
    swapped = np.concatenate([w[2 * c:4 * c], w[:2 * c], w[4 * c:]], axis=0)
    q = dict(p, z=np.transpose(p["z"], (1, 0, 2)).copy(), w_in=swapped)
    y_in = TM.trimul_fwd(**p, incoming=True)["y"]
    y_out_t = np.transpose(TM.trimul_fwd(**q, incoming=False)["y"], (1, 0, 2))
    assert np.max(np.abs(y_in - y_out_t)) <= 1e-12 * np.max(np.abs(y_in))
    # and the two directions really differ on these inputs
    assert np.max(np.abs(y_in - TM.trimul_fwd(**p, incoming=False)["y"])) > 1e-3


def test_closed_forms():
    p, _ = params(4, 8, 6, seed=13)
    c = p["w_out"].shape[1]
    # W_ap = 0: a = 0, t = 0, LayerNorm(0) = beta_out, so y = g * (beta_out W_o^T)
    q = dict(p)
    q["w_in"] = p["w_in"].copy()
    q["w_in"][:c] = 0.0
    f = TM.trimul_fwd(**q)
    assert np.max(np.abs(f["t"])) == 0.0
    want = f["g"] * (p["beta_out"] @ p["w_out"].T)
    assert np.max(np.abs(f["y"] - want)) <= 1e-12
    # N = 1: the only third token is the pair itself, t = a * b (both directions)
    p1, _ = params(1, 8, 6, seed=14)
    for incoming in (False, True):
        f = TM.trimul_fwd(**p1, incoming=incoming)
        assert np.max(np.abs(f["t"] - f["a"] * f["b"])) <= 1e-14
