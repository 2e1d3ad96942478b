"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar (normwise max|x - ref| / max|ref| per output tensor): 1e-4 for fp32 runs,
2e-2 for bf16 inputs/outputs with fp32 accumulation.  Results must also be
bitwise identical across repeated calls.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import triangle_attention_tri_amd as ta
from triangle_attention_tri_amd import inputs
from tests.helpers import assert_close, assert_lse, lse_tol, np64

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
OUT_KEYS = ("out", "attn", "lse")
GRAD_KEYS = ("dq", "dk", "dv", "dbias", "dgate")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x, device):
    return {k: (None if v is None else v.to(device)) for k, v in x.items()}


def run_gpu(x, ending=False):
    out, attn, lse = ta.fwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], x["mask"], ending)
    dq, dk, dv, dbias, dgate = ta.bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], x["mask"], attn, lse,
                                      x["dout"], ending)
    torch.cuda.synchronize()
    return dict(out=out, attn=attn, lse=lse, dq=dq, dk=dk, dv=dv, dbias=dbias, dgate=dgate)


# --- kernel-order views (rows i first) of caller tensors for either node -----
def k_qkv(t, ending):   # caller [a,H,b,c] -> kernel [i,H,j,c]
    return t.permute(2, 1, 0, 3) if ending else t


def k_pair(t, ending):  # caller [a,b,H,c] -> kernel [i,j,H,c]
    return t.permute(1, 0, 2, 3) if ending else t


def k_bias(t, ending):  # caller [H,x,y] -> kernel [H,j,k]
    return t.permute(0, 2, 1) if ending else t


def k_mask(t, ending):
    return None if t is None else (t.t() if ending else t)


def oracle_rows(xc, rows, ending):
    """Oracle forward+backward for the kernel rows `rows` (all queries, all keys)."""
    q = k_qkv(xc["q"], ending)[rows]
    k = k_qkv(xc["k"], ending)[rows]
    v = k_qkv(xc["v"], ending)[rows]
    gate = k_pair(xc["gate"], ending)[rows]
    dout = k_pair(xc["dout"], ending)[rows]
    bias = k_bias(xc["bias"], ending)
    mask = k_mask(xc["mask"], ending)
    mask = None if mask is None else mask[rows]
    return oracle.attn_bwd(q, k, v, bias, gate, mask, dout)


def oracle_dbias_queries(xc, qsel, ending):
    """Exact dbias[:, qsel, :] (kernel order) summed over every row."""
    q = k_qkv(xc["q"], ending)[:, :, qsel]
    gate = k_pair(xc["gate"], ending)[:, qsel]
    dout = k_pair(xc["dout"], ending)[:, qsel]
    bias = k_bias(xc["bias"], ending)[:, qsel]
    return oracle.attn_bwd(q, k_qkv(xc["k"], ending), k_qkv(xc["v"], ending), bias, gate,
                           k_mask(xc["mask"], ending), dout)["dbias"]


def gpu_rows(res, rows, ending):
    g = {k: v.cpu() for k, v in res.items()}
    return dict(out=k_pair(g["out"], ending)[rows], attn=g["attn"][rows], lse=g["lse"][rows],
                dq=k_qkv(g["dq"], ending)[rows], dk=k_qkv(g["dk"], ending)[rows], dv=k_qkv(g["dv"], ending)[rows],
                dgate=k_pair(g["dgate"], ending)[rows], dbias=k_bias(g["dbias"], ending))


def check_full(name, xc, res, tol, ending=False):
    n = xc["q"].shape[0]
    rows = list(range(n))
    ref = oracle_rows(xc, rows, ending)
    got = gpu_rows(res, rows, ending)
    errs = {}
    for key in OUT_KEYS + GRAD_KEYS:
        if key == "lse":
            errs[key] = assert_lse(f"{name}:lse", got[key], ref[key], lse_tol(tol))
        else:
            errs[key] = assert_close(f"{name}:{key}", got[key], ref[key], tol)
    log(name, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return errs


def check_sampled(name, xc, res, tol, ending, rows, qsel):
    ref = oracle_rows(xc, rows, ending)
    got = gpu_rows(res, rows, ending)
    errs = {}
    for key in OUT_KEYS + ("dq", "dk", "dv", "dgate"):
        if key == "lse":
            errs[key] = assert_lse(f"{name}:lse", got[key], ref[key], lse_tol(tol))
        else:
            errs[key] = assert_close(f"{name}:{key}", got[key], ref[key], tol)
    db_ref = oracle_dbias_queries(xc, qsel, ending)
    errs["dbias"] = assert_close(f"{name}:dbias", got["dbias"][:, qsel], db_ref, tol)
    log(name, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    return errs


# --------------------------------------------------------------------------- workloads
@pytest.mark.parametrize("widx", [0, 1, 2])
def test_workload_full(device, widx):
    w = inputs.WORKLOADS[widx]
    log(f"workload {widx} {w.name}: full oracle comparison")
    xc = inputs.workload_inputs(widx)
    res = run_gpu(to_dev(xc, device))
    check_full(w.name, xc, res, w.tol)


@pytest.mark.parametrize("node", ["start", "end"])
def test_workload3_sampled(device, node):
    w = inputs.WORKLOADS[3]
    log(f"workload 3 {w.name} node={node}: sampled rows / dbias queries")
    xc = inputs.workload_inputs(3)
    ending = node == "end"
    res = run_gpu(to_dev(xc, device), ending)
    n = w.n
    rng = np.random.default_rng(3)
    rows = sorted({0, 1, n // 2, n - 1, *rng.choice(n, 4, replace=False).tolist()})
    qsel = sorted({0, 31, 32, n - 1, *rng.choice(n, 4, replace=False).tolist()})
    check_sampled(f"{w.name}:{node}", xc, res, w.tol, ending, rows, qsel)


@pytest.mark.parametrize("node", ["start", "end"])
def test_attention_n768_sampled(device, node):
    """Attention at the measured size (N=768, H=4, c=32, bf16), both nodes."""
    log(f"attention n=768 node={node}: sampled rows / dbias queries")
    xc = inputs.attn_inputs(768, 4, 32, torch.bfloat16, seed=4)
    ending = node == "end"
    res = run_gpu(to_dev(xc, device), ending)
    rng = np.random.default_rng(4)
    rows = sorted({0, 383, 767, *rng.choice(768, 3, replace=False).tolist()})
    qsel = sorted({0, 767, *rng.choice(768, 4, replace=False).tolist()})
    check_sampled(f"n768:{node}", xc, res, 2e-2, ending, rows, qsel)


# --------------------------------------------------------------------------- edge cases
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [1, 2, 3, 17, 33, 65, 127])
def test_ragged_sizes(device, n, dtype):
    log(f"ragged n={n} dtype={dtype}")
    xc = inputs.attn_inputs(n, 4, 32, dtype, seed=100 + n, bias_std=1.5)
    if n >= 3:
        xc["mask"] = inputs.random_mask(n, seed=n, p_keep=0.7, full_rows=(1,))
    res = run_gpu(to_dev(xc, device))
    check_full(f"ragged{n}", xc, res, TOL[dtype])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ending_node_small(device, dtype):
    n = 45
    log(f"ending node n={n} dtype={dtype}")
    xc = inputs.attn_inputs(n, 4, 32, dtype, seed=7, bias_std=2.0)
    xc["mask"] = inputs.random_mask(n, seed=9, p_keep=0.8, full_rows=(4,))
    res = run_gpu(to_dev(xc, device), ending=True)
    check_full(f"end{n}", xc, res, TOL[dtype], ending=True)


def test_row_slices(device):
    """n_rows < n through the C ABI: a row slice gives that slice's outputs and dbias partial."""
    n, h = 70, 4
    log(f"row slices n={n}")
    xc = inputs.attn_inputs(n, h, 32, torch.bfloat16, seed=11)
    xd = to_dev(xc, device)
    full = run_gpu(xd)
    r0, r1 = 13, 50
    sl = {k: (None if v is None else (v if k == "bias" else v[r0:r1].contiguous())) for k, v in xd.items()}
    part = run_gpu(sl)
    for key in ("out", "attn", "lse", "dq", "dk", "dv", "dgate"):
        assert torch.equal(part[key], full[key][r0:r1]), key
    ref = oracle.attn_bwd(xc["q"][r0:r1], xc["k"][r0:r1], xc["v"][r0:r1], xc["bias"], xc["gate"][r0:r1], None,
                          xc["dout"][r0:r1])
    assert_close("slice dbias", part["dbias"], ref["dbias"], 2e-2)


def test_row_slice_key_ranges(device):
    """bf16 with several key ranges and a row count that is not a multiple of the row group:
    n = 200 splits the keys into two ranges of four tiles, and 37 rows leave the last group of
    four with one live row (padded rows, padded dQ partials).  Each row's outputs match the full
    run bit for bit; the slice's dbias matches the oracle.  On a 256-CU device the 37-row slice
    launches the one-row forward form (its two-row grid would not fill the device) and the full
    call the two-row form, so this also checks that the two forms agree bit for bit."""
    n, h = 200, 4
    log(f"row slice with key ranges n={n}")
    xc = inputs.attn_inputs(n, h, 32, torch.bfloat16, seed=12)
    xd = to_dev(xc, device)
    full = run_gpu(xd)
    r0, r1 = 5, 42
    sl = {k: (None if v is None else (v if k == "bias" else v[r0:r1].contiguous())) for k, v in xd.items()}
    part = run_gpu(sl)
    for key in ("out", "attn", "lse", "dq", "dk", "dv", "dgate"):
        assert torch.equal(part[key], full[key][r0:r1]), key
    ref = oracle.attn_bwd(xc["q"][r0:r1], xc["k"][r0:r1], xc["v"][r0:r1], xc["bias"], xc["gate"][r0:r1], None,
                          xc["dout"][r0:r1])
    for key in ("dq", "dk", "dv", "dbias"):
        assert_close(f"slice {key}", part[key], ref[key], 2e-2)


def test_masked_keys_bitwise(device):
    """Randomising k, v and bias at masked keys leaves every output bit-identical."""
    n = 96
    log("masked keys bitwise")
    xc = inputs.attn_inputs(n, 4, 32, torch.bfloat16, seed=21)
    mask = torch.ones((n, n), dtype=torch.uint8)
    dead_keys = [5, 40, 41, 90]
    mask[:, dead_keys] = 0
    xc["mask"] = mask
    base = run_gpu(to_dev(xc, device))
    x2 = dict(xc)
    g = torch.Generator().manual_seed(5)
    for name in ("k", "v"):
        t = x2[name].clone()
        t[:, :, dead_keys] = torch.randn(t[:, :, dead_keys].shape, generator=g).to(t.dtype) * 10
        x2[name] = t
    b = x2["bias"].clone()
    b[:, :, dead_keys] = torch.randn(b[:, :, dead_keys].shape, generator=g).to(b.dtype) * 10
    x2["bias"] = b
    res = run_gpu(to_dev(x2, device))
    for key in ("out", "attn", "lse", "dq", "dgate"):
        assert torch.equal(res[key], base[key]), key
    assert torch.all(res["dk"][:, :, dead_keys] == 0) and torch.all(res["dv"][:, :, dead_keys] == 0)
    assert torch.all(res["dbias"][:, :, dead_keys] == 0)


def test_constant_values(device):
    """V constant along keys: every softmax row sums to one, so attn equals that constant."""
    n = 80
    xc = inputs.attn_inputs(n, 4, 32, torch.float32, seed=31, bias_std=2.0)
    u = torch.randn(32, generator=torch.Generator().manual_seed(1))
    xc["v"] = u.expand(n, 4, n, 32).contiguous()
    res = run_gpu(to_dev(xc, device))
    err = (res["attn"].cpu() - u).abs().max().item()
    assert err < 1e-5, err


@pytest.mark.parametrize("widx", [1, 2])
def test_determinism(device, widx):
    """Five repeated calls give bitwise identical outputs and gradients."""
    log(f"determinism workload {widx}")
    xd = to_dev(inputs.workload_inputs(widx), device)
    first = run_gpu(xd)
    for rep in range(4):
        again = run_gpu(xd)
        for key in first:
            assert torch.equal(first[key], again[key]), f"repeat {rep}: {key}"


def test_determinism_n768(device):
    log("determinism n=768 (5 runs)")
    xd = to_dev(inputs.attn_inputs(768, 4, 32, torch.bfloat16, seed=4), device)
    first = run_gpu(xd)
    for rep in range(4):
        again = run_gpu(xd)
        for key in first:
            assert torch.equal(first[key], again[key]), f"repeat {rep}: {key}"


# --------------------------------------------------------------------------- other paths
@pytest.mark.parametrize("n,dtype", [(300, torch.float32), (960, torch.bfloat16), (736, torch.float32)])
def test_row_group_backward_sizes(device, n, dtype):
    """Largest sizes of each backward path: fp32 past the per-row tile kernel's limit
    (n > 256) takes the fallback rows kernel; bf16 n = 960 (the largest accepted) runs the
    group kernel with eight key ranges."""
    assert n <= ta.max_n(dtype)
    log(f"row-group backward n={n} dtype={dtype}")
    xc = inputs.attn_inputs(n, 4, 32, dtype, seed=200 + n, bias_std=1.5)
    xc["mask"] = inputs.random_mask(n, seed=n, p_keep=0.85, full_rows=(2,))
    res = run_gpu(to_dev(xc, device))
    rng = np.random.default_rng(n)
    rows = sorted({0, 2, n // 2, n - 1, *rng.choice(n, 3, replace=False).tolist()})
    qsel = sorted({0, 31, n - 1, *rng.choice(n, 3, replace=False).tolist()})
    check_sampled(f"rows{n}", xc, res, TOL[dtype], False, rows, qsel)


def test_autograd_function(device):
    """torch.autograd through TriAttnFunction gives the C ABI's gradients."""
    from triangle_attention_tri_amd.autograd import tri_attn
    n = 40
    log("autograd function")
    xc = inputs.attn_inputs(n, 4, 32, torch.bfloat16, seed=41)
    xc["mask"] = inputs.random_mask(n, seed=3, p_keep=0.8)
    xd = to_dev(xc, device)
    leaves = {k: xd[k].clone().requires_grad_(True) for k in ("q", "k", "v", "bias", "gate")}
    out = tri_attn(leaves["q"], leaves["k"], leaves["v"], leaves["bias"], leaves["gate"], xd["mask"])
    out.backward(xd["dout"])
    torch.cuda.synchronize()
    ref = oracle_rows(xc, list(range(n)), False)
    assert_close("autograd out", out.detach().cpu(), ref["out"], 2e-2)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("bias", "dbias"), ("gate", "dgate")):
        assert_close(f"autograd {key}", leaves[name].grad.cpu(), ref[key], 2e-2)


def test_large_bias(device):
    """bf16 with a wide pair bias (std 30, |b| up to ~130): the bias term enters through MFMAs with
    sqrt(c) held in bf16 (relative error 1.1e-4 of the term), still inside the bf16 bar."""
    n = 96
    xc = inputs.attn_inputs(n, 4, 32, torch.bfloat16, seed=5, bias_std=30.0)
    log(f"large bias n={n}: max |b| = {xc['bias'].float().abs().max().item():.1f}")
    res = run_gpu(to_dev(xc, device))
    check_full("bias_std30", xc, res, TOL[torch.bfloat16])


def test_profiled_stage_events(device):
    """tri_attn_bwd_profiled with some stage events NULL gives tri_attn_bwd's results bit for bit and
    times the stages it was given events for."""
    import ctypes
    n = 128
    xc = inputs.attn_inputs(n, 4, 32, torch.bfloat16, seed=3)
    x = to_dev(xc, device)
    out, attn, lse = ta.fwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], None)
    ref = ta.bwd(x["q"], x["k"], x["v"], x["bias"], x["gate"], None, attn, lse, x["dout"])
    lib = ta.load()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p() for _ in range(2)]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    stage = (ctypes.c_void_p * 4)(None, ev[0], ev[1], None)
    ws = torch.empty(ta.workspace_size(n, n, 4, 32, torch.bfloat16), dtype=torch.uint8, device=device)
    outs = [torch.empty_like(t) for t in ref]
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    lib.tri_attn_bwd_profiled.argtypes = list(lib.tri_attn_bwd.argtypes) + [ctypes.c_void_p]
    lib.tri_attn_bwd_profiled.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    st = lib.tri_attn_bwd_profiled(n, n, 4, 32, ta.BF16, 0, P(x["q"]), P(x["k"]), P(x["v"]), P(x["bias"]),
                                   P(x["gate"]), None, P(attn), P(lse), P(x["dout"]), *[P(t) for t in outs], P(ws),
                                   ctypes.c_size_t(ws.numel()), stream, ctypes.cast(stage, ctypes.c_void_p))
    assert st == 0, st
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)
    ms = ctypes.c_float()
    assert hip.hipEventSynchronize(ev[1]) == 0
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    log(f"main backward kernel at n={n}: {ms.value:.3f} ms")
    assert ms.value > 0.0


@pytest.mark.parametrize("case", ["bf16_n768_start", "bf16_n256_end_mask", "fp32_n300_rows"])
def test_backward_chunking_bitwise(device, case, monkeypatch):
    """The backward runs its rows in chunks (tri_attn_bwd_chunk_rows) that carry the pair-bias gradient as an fp32
    running sum in a single pass's order.  Every output is bit for bit that of one pass over all rows (and of
    32-row chunks), for the bf16 row-group kernel at both nodes and for the fp32 rows kernel."""
    n, dtype, ending, mask = {"bf16_n768_start": (768, torch.bfloat16, False, None),
                              "bf16_n256_end_mask": (256, torch.bfloat16, True, "random"),
                              "fp32_n300_rows": (300, torch.float32, False, "random")}[case]
    xc = inputs.attn_inputs(n, 4, 32, dtype, seed=77, bias_std=1.5)
    if mask:
        xc["mask"] = inputs.random_mask(n, seed=78, p_keep=0.8, full_rows=(3,))
    xd = to_dev(xc, device)
    monkeypatch.delenv("TRI_ATTN_BWD_CHUNK_ROWS", raising=False)
    default_chunk = ta.bwd_chunk_rows(n, n, 4, 32, dtype)
    base = run_gpu(xd, ending)
    for forced in (n, 32):
        monkeypatch.setenv("TRI_ATTN_BWD_CHUNK_ROWS", str(forced))
        assert ta.bwd_chunk_rows(n, n, 4, 32, dtype) == forced
        res = run_gpu(xd, ending)
        for key in base:
            assert torch.equal(res[key], base[key]), f"{case}: {key} differs with {forced}-row chunks " \
                                                     f"(default {default_chunk})"
    log(f"{case}: default chunk {default_chunk}, one pass and 32-row chunks bitwise equal")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("node", ["start", "end"])
def test_largest_bf16_size(device, node):
    """bf16 at the largest accepted n (2048: the forward's table of kept-key words per workgroup holds 64 key
    tiles), H=2, with a key mask that drops a whole row: sixteen key ranges, 32-row backward chunks, sampled rows
    and exact dbias columns against the oracle, at both nodes."""
    n, h = ta.max_n(torch.bfloat16), 2
    assert n == 2048
    log(f"largest bf16 size n={n} h={h} node={node}")
    xc = inputs.attn_inputs(n, h, 32, torch.bfloat16, seed=2048, bias_std=1.5)
    xc["mask"] = inputs.random_mask(n, seed=2049, p_keep=0.9, full_rows=(5,))
    ending = node == "end"
    res = run_gpu(to_dev(xc, device), ending)
    rng = np.random.default_rng(2048)
    rows = sorted({0, 5, n // 2, n - 1, *rng.choice(n, 2, replace=False).tolist()})
    qsel = sorted({0, 31, n - 1, *rng.choice(n, 2, replace=False).tolist()})
    check_sampled(f"n{n}:{node}", xc, res, 2e-2, ending, rows, qsel)
