"""GPU parity of the block around the attention: LayerNorm + projection front end
and the output linear, forward and backward, through the C ABI, against the
fp64 oracle (oracle/block.py).  Bar: normwise 2e-2 (bf16 inputs/outputs, fp32
accumulation); the LayerNorm statistics (fp32 outputs) 1e-5.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import block as B
import triangle_attention_tri_amd as ta
from triangle_attention_tri_amd import inputs
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu
H, C, CZ = 4, 32, 128
TOL = 2e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, device):
    return {k: v.to(device) for k, v in x.items()}


def check_front_fwd(n, seed, device, affine=True):
    x = inputs.block_inputs(n, seed=seed, affine=affine)
    xd = dev(x, device)
    q, k, v, gate, bias, mean, rstd = ta.ln_proj_fwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"])
    torch.cuda.synchronize()
    ref = B.ln_proj_fwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], H, C)
    for name, got in dict(q=q, k=k, v=v, gate=gate, bias=bias).items():
        assert_close(f"n{n}:{name}", got.cpu(), ref[name], TOL)
    assert_close(f"n{n}:mean", mean.cpu(), ref["mean"], 1e-5)
    assert_close(f"n{n}:rstd", rstd.cpu(), ref["rstd"], 1e-5)
    return x, xd, (q, k, v, gate, bias, mean, rstd)


@pytest.mark.parametrize("n", [1, 5, 37, 64])
def test_ln_proj_fwd(device, n):
    log(f"ln_proj_fwd n={n}")
    check_front_fwd(n, seed=10 + n, device=device)


@pytest.mark.parametrize("n", [1, 5, 37, 64])
def test_ln_proj_bwd(device, n):
    log(f"ln_proj_bwd n={n}")
    x = inputs.block_inputs(n, seed=20 + n, affine=True)
    gr = inputs.proj_grad_inputs(n, seed=30 + n)
    xd, gd = dev(x, device), dev(gr, device)
    _, _, _, _, _, mean, rstd = ta.ln_proj_fwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"])
    got = ta.ln_proj_bwd(xd["z"], xd["gamma"], xd["beta"], mean, rstd, xd["w_qkvg"], xd["w_bias"], gd["dq"], gd["dk"],
                         gd["dv"], gd["dgate"], gd["dbias"])
    torch.cuda.synchronize()
    ref = B.ln_proj_bwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], gr["dq"], gr["dk"], gr["dv"],
                        gr["dgate"], gr["dbias"], H, C)
    errs = {}
    for name, t in zip(("dz", "dgamma", "dbeta", "dw_qkvg", "dw_bias"), got):
        errs[name] = assert_close(f"n{n}:{name}", t.cpu(), ref[name], TOL)
    log(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("n", [1, 7, 40])
def test_out_proj(device, n):
    log(f"out_proj n={n}")
    g = torch.Generator().manual_seed(40 + n)
    o = torch.randn((n, n, H, C), generator=g).bfloat16()
    w_o = (torch.randn((CZ, H * C), generator=g) / 128 ** 0.5).bfloat16()
    dy = torch.randn((n, n, CZ), generator=g).bfloat16()
    od, wd, dyd = o.to(device), w_o.to(device), dy.to(device)
    y = ta.out_proj_fwd(od, wd)
    d_o, dw_o = ta.out_proj_bwd(od, wd, dyd)
    torch.cuda.synchronize()
    assert_close("y", y.cpu(), B.out_proj_fwd(o, w_o), TOL)
    ref = B.out_proj_bwd(o, w_o, dy)
    assert_close("do", d_o.cpu(), ref["do"], TOL)
    assert_close("dw_o", dw_o.cpu(), ref["dw_o"], TOL)


@pytest.mark.parametrize("ending", [False, True])
def test_block_small(device, ending):
    """The whole block (front end -> attention -> output linear), forward and backward."""
    n = 48
    log(f"block n={n} ending={ending}")
    x = inputs.block_inputs(n, seed=50, affine=True)
    xd = dev(x, device)
    y, saved = ta.block_fwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"], ending=ending)
    grads = ta.block_bwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"], saved, xd["dy"],
                         ending=ending)
    torch.cuda.synchronize()
    ref = B.block_bwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], x["w_o"], x["dy"], H, C, ending=ending)
    errs = {"y": assert_close("y", y.cpu(), ref["y"], TOL)}
    for name in ("dz", "dgamma", "dbeta", "dw_qkvg", "dw_bias", "dw_o"):
        errs[name] = assert_close(name, grads[name].cpu(), ref[name], TOL)
    log(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_front_end_n768(device):
    """Front end forward and backward at the block's full size (N=768, c_z=128), every output."""
    n = 768
    log("front end n=768")
    x = inputs.block_inputs(n, seed=4)
    gr = inputs.proj_grad_inputs(n, seed=6)
    xd, gd = dev(x, device), dev(gr, device)
    q, k, v, gate, bias, mean, rstd = ta.ln_proj_fwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"])
    got = ta.ln_proj_bwd(xd["z"], xd["gamma"], xd["beta"], mean, rstd, xd["w_qkvg"], xd["w_bias"], gd["dq"], gd["dk"],
                         gd["dv"], gd["dgate"], gd["dbias"])
    torch.cuda.synchronize()
    ref = B.ln_proj_fwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], H, C)
    for name, t in dict(q=q, k=k, v=v, gate=gate, bias=bias).items():
        assert_close(f"n768:{name}", t.cpu(), ref[name], TOL)
    del ref
    ref = B.ln_proj_bwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], gr["dq"], gr["dk"], gr["dv"],
                        gr["dgate"], gr["dbias"], H, C)
    for name, t in zip(("dz", "dgamma", "dbeta", "dw_qkvg", "dw_bias"), got):
        assert_close(f"n768:{name}", t.cpu(), ref[name], TOL)


def test_block_determinism(device):
    n = 96
    log("block determinism")
    xd = dev(inputs.block_inputs(n, seed=60, affine=True), device)
    runs = []
    for _ in range(3):
        y, saved = ta.block_fwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"])
        g = ta.block_bwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"], saved, xd["dy"])
        runs.append(dict(y=y, **g))
    torch.cuda.synchronize()
    for r in runs[1:]:
        for key in runs[0]:
            assert torch.equal(runs[0][key], r[key]), key


def test_block_fwd_chunked(device):
    """Chunked inference of the starting-node block: y is bit for bit the unchunked block's for chunks that
    divide n, do not divide it and are single rows, and matches the block oracle; a budget picks the largest
    chunk whose workspace fits."""
    n = 96
    x = inputs.block_inputs(n, seed=51, affine=True)
    x["mask"] = inputs.random_mask(n, seed=52, p_keep=0.8, full_rows=(5,))
    xd = dev(x, device)
    w = (xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"])
    y_full, _ = ta.block_fwd(*w, mask=xd["mask"])
    torch.cuda.synchronize()
    ref = B.block_fwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], x["w_o"], H, C, mask=x["mask"])
    e = assert_close("y(unchunked)", y_full.cpu(), ref["y"], TOL)
    log(f"chunked block n={n}: unchunked y error {e:.2e}")
    sizes = {}
    for rows in (n, 32, 37, 1):
        y, r, need = ta.block_fwd_chunked(*w, mask=xd["mask"], rows_per_chunk=rows)
        torch.cuda.synchronize()
        assert r == rows
        assert torch.equal(y, y_full), f"rows_per_chunk={rows}: y differs from the unchunked block"
        sizes[rows] = need
        log(f"  rows_per_chunk={rows}: workspace {need / 2**20:.2f} MiB, bitwise equal")
    y, r, need = ta.block_fwd_chunked(*w, mask=xd["mask"], budget_bytes=sizes[37] + 100)
    torch.cuda.synchronize()
    assert r >= 37 and need <= sizes[37] + 100 and torch.equal(y, y_full)


@pytest.mark.parametrize("n,masked", [(96, True), (130, False), (37, True)])
def test_block_fwd_fused(device, n, masked):
    """Fused inference of the starting-node block (LayerNorm, q and the gate projected inside the attention
    kernel): y is bit for bit the chunked forward's for whole, uneven and single-row chunks (ragged n and a fully
    masked row included), and matches the block oracle."""
    x = inputs.block_inputs(n, seed=61 + n, affine=True)
    if masked:
        x["mask"] = inputs.random_mask(n, seed=62 + n, p_keep=0.8, full_rows=(3,))
    xd = dev(x, device)
    w = (xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"])
    mask = xd.get("mask")
    y_ref, _, _ = ta.block_fwd_chunked(*w, mask=mask, rows_per_chunk=n)
    torch.cuda.synchronize()
    ref = B.block_fwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], x["w_o"], H, C, mask=x.get("mask"))
    for rows in (n, 32, 1):
        y, need = ta.block_fwd_fused(*w, mask=mask, rows_per_chunk=rows)
        torch.cuda.synchronize()
        e = assert_close(f"y(fused, rows {rows})", y.cpu(), ref["y"], TOL)
        assert torch.equal(y, y_ref), f"n={n} rows_per_chunk={rows}: fused y differs from the chunked forward"
        log(f"fused block n={n} rows={rows}: error {e:.2e}, workspace {need / 2**20:.2f} MiB, bitwise equal")


@pytest.mark.parametrize("n", [768])
def test_block_fwd_fused_n768(device, n):
    """The fused inference block at the benchmark's size, bitwise against the chunked forward."""
    x = inputs.block_inputs(n, seed=68, affine=True)
    xd = dev(x, device)
    w = (xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"])
    y_ref, _, _ = ta.block_fwd_chunked(*w, rows_per_chunk=n)
    y, _ = ta.block_fwd_fused(*w)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)


def test_out_proj_n768(device):
    """Output linear forward and backward at the block's full size (768 x 768 = 589,824 pairs): the persistent
    multi-tile loop, the cross-tile prefetch and the per-workgroup weight-gradient partials all run here."""
    n = 768
    log(f"out_proj n={n} ({n * n} pairs)")
    g = torch.Generator().manual_seed(768)
    o = torch.randn((n, n, H, C), generator=g).bfloat16()
    w_o = (torch.randn((CZ, H * C), generator=g) / 128 ** 0.5).bfloat16()
    dy = torch.randn((n, n, CZ), generator=g).bfloat16()
    od, wd, dyd = o.to(device), w_o.to(device), dy.to(device)
    y = ta.out_proj_fwd(od, wd)
    d_o, dw_o = ta.out_proj_bwd(od, wd, dyd)
    torch.cuda.synchronize()
    errs = {"y": assert_close("y", y.cpu(), B.out_proj_fwd(o, w_o), TOL)}
    ref = B.out_proj_bwd(o, w_o, dy)
    errs["do"] = assert_close("do", d_o.cpu(), ref["do"], TOL)
    errs["dw_o"] = assert_close("dw_o", dw_o.cpu(), ref["dw_o"], TOL)
    log(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ending", [False, True])
def test_block_n768(device, ending):
    """The whole block at its full size (z [768, 768, 128] bf16, H=4, c=32, c_z=128): front end -> attention
    (starting or ending node) -> output linear, forward and backward, in the launch configuration the benchmark
    times.  Every element of y, dz, dgamma, dbeta, dw_qkvg, dw_bias and dw_o is compared with the fp64 block
    oracle (the oracle runs the full attention forward and backward over all 768 rows)."""
    n = 768
    log(f"block n={n} ending={ending}: GPU")
    x = inputs.block_inputs(n, seed=4, affine=True)
    xd = dev(x, device)
    y, saved = ta.block_fwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"], ending=ending)
    grads = ta.block_bwd(xd["z"], xd["gamma"], xd["beta"], xd["w_qkvg"], xd["w_bias"], xd["w_o"], saved, xd["dy"],
                         ending=ending)
    torch.cuda.synchronize()
    got = {"y": y.cpu(), **{k: v.cpu() for k, v in grads.items()}}
    del saved, grads, y, xd
    torch.cuda.empty_cache()
    log(f"block n={n} ending={ending}: oracle")
    ref = B.block_bwd(x["z"], x["gamma"], x["beta"], x["w_qkvg"], x["w_bias"], x["w_o"], x["dy"], H, C, ending=ending)
    errs = {}
    for name in ("y", "dz", "dgamma", "dbeta", "dw_qkvg", "dw_bias", "dw_o"):
        errs[name] = assert_close(name, got[name], ref[name], TOL)
    log(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))
