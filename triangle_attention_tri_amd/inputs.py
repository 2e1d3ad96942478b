"""Seeded synthetic inputs for the triangle-attention workloads.

This module holds no arithmetic of the method: it only draws random tensors
and builds masks, so the GPU path and the oracle can be fed the same values.

Recipe (all on the CPU, one ``torch.Generator`` per call, seeded with the
workload index):
* draw order q, k, v, bias, gate, dout, each standard normal float32 in the
  boundary layouts (q, k, v [N,H,N,c]; bias [H,N,N]; gate, dout [N,N,H,c]);
* bias is multiplied by ``bias_std`` (2 for the wide-bias workload);
* bf16 workloads round the float32 draws to bfloat16 (round to nearest even);
  the oracle consumes the rounded values;
* the key-padding workload keeps keys k < valid_len for every row i
  (mask[i, k] = 1), i.e. the trailing tokens are padding.
The sizes mirror the crops the pages train at (TurboPairFormer news item,
"Benchmark di addestramento": crops 384, 640, 768) plus the AlphaFold2
initial-training crop 256 and a small fp32 case; no dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    n: int
    h: int = 4
    c: int = 32
    dtype: torch.dtype = torch.bfloat16
    bias_std: float = 1.0
    valid_len: int | None = None
    nodes: tuple = ("start",)
    block: bool = False
    cz: int = 128
    tol: float = 2e-2


WORKLOADS = {
    0: Workload(0, "start_n64_h4_c32_fp32", 64, dtype=torch.float32, tol=1e-4),
    1: Workload(1, "start_n256_h4_c32_bf16", 256),
    2: Workload(2, "start_n384_h4_c32_bf16_keymask345", 384, valid_len=345),
    3: Workload(3, "start_end_n640_h4_c32_bf16_bias_std2", 640, bias_std=2.0, nodes=("start", "end")),
    4: Workload(4, "block_start_end_n768_h4_c32_cz128_bf16", 768, nodes=("start", "end"), block=True),
}


def attn_inputs(n: int, h: int = 4, c: int = 32, dtype=torch.bfloat16, seed: int = 0,
                bias_std: float = 1.0, valid_len: int | None = None) -> dict:
    """Seeded attention inputs (CPU tensors).  See the module docstring."""
    g = torch.Generator().manual_seed(int(seed))
    q = torch.randn((n, h, n, c), generator=g)
    k = torch.randn((n, h, n, c), generator=g)
    v = torch.randn((n, h, n, c), generator=g)
    bias = torch.randn((h, n, n), generator=g)
    if bias_std != 1.0:
        bias = bias * bias_std
    gate = torch.randn((n, n, h, c), generator=g)
    dout = torch.randn((n, n, h, c), generator=g)
    out = dict(q=q, k=k, v=v, bias=bias, gate=gate, dout=dout)
    if dtype != torch.float32:
        out = {key: t.to(dtype) for key, t in out.items()}
    mask = None
    if valid_len is not None:
        mask = torch.zeros((n, n), dtype=torch.uint8)
        mask[:, :valid_len] = 1
    out["mask"] = mask
    return out


def workload_inputs(index: int) -> dict:
    w = WORKLOADS[index]
    return attn_inputs(w.n, w.h, w.c, w.dtype, seed=w.index, bias_std=w.bias_std, valid_len=w.valid_len)


def random_mask(n: int, seed: int, p_keep: float = 0.7, full_rows: tuple = ()) -> torch.Tensor:
    """Random keep/drop mask [n, n] (uint8); rows listed in full_rows are all dropped."""
    g = torch.Generator().manual_seed(int(seed))
    m = (torch.rand((n, n), generator=g) < p_keep).to(torch.uint8)
    for r in full_rows:
        m[r, :] = 0
    return m


def block_inputs(n: int, cz: int = 128, h: int = 4, c: int = 32, dtype=torch.bfloat16, seed: int = 4,
                 affine: bool = False) -> dict:
    """Seeded inputs of the LayerNorm + projections + attention + output-linear block.

    Draw order: z [n,n,cz] ~ N(0,1); w_qkvg [4*h*c, cz], w_bias [h, cz] and
    w_o [cz, h*c] ~ N(0, 1/cz) (standard deviation 1/sqrt(cz)); dy [n,n,cz] ~ N(0,1).
    gamma = 1 and beta = 0 unless ``affine`` (then gamma ~ 1 + 0.1 N(0,1) and
    beta ~ 0.1 N(0,1), drawn last), so that tests can see both LayerNorm
    parameters act.  bf16 rounds every tensor (the oracle reads the rounded
    values); gamma and beta are kept in the same dtype.
    """
    g = torch.Generator().manual_seed(int(seed))
    z = torch.randn((n, n, cz), generator=g)
    w_qkvg = torch.randn((4 * h * c, cz), generator=g) / cz ** 0.5
    w_bias = torch.randn((h, cz), generator=g) / cz ** 0.5
    w_o = torch.randn((cz, h * c), generator=g) / (h * c) ** 0.5
    dy = torch.randn((n, n, cz), generator=g)
    if affine:
        gamma = 1.0 + 0.1 * torch.randn(cz, generator=g)
        beta = 0.1 * torch.randn(cz, generator=g)
    else:
        gamma, beta = torch.ones(cz), torch.zeros(cz)
    out = dict(z=z, w_qkvg=w_qkvg, w_bias=w_bias, w_o=w_o, dy=dy, gamma=gamma, beta=beta)
    if dtype != torch.float32:
        out = {key: t.to(dtype) for key, t in out.items()}
    return out


def proj_grad_inputs(n: int, h: int = 4, c: int = 32, dtype=torch.bfloat16, seed: int = 5) -> dict:
    """Seeded upstream gradients of the front end's five outputs, each ~ N(0,1):
    dq, dk, dv [n,h,n,c], dgate [n,n,h,c], dbias [h,n,n], drawn in that order."""
    g = torch.Generator().manual_seed(int(seed))
    out = dict(dq=torch.randn((n, h, n, c), generator=g), dk=torch.randn((n, h, n, c), generator=g),
               dv=torch.randn((n, h, n, c), generator=g), dgate=torch.randn((n, n, h, c), generator=g),
               dbias=torch.randn((h, n, n), generator=g))
    return {key: t.to(dtype) for key, t in out.items()}


def trimul_inputs(n: int, cz: int = 128, c: int = 128, dtype=torch.bfloat16, seed: int = 7) -> dict:
    """Seeded inputs of the triangular multiplicative update.

    Draw order: z [n,n,cz] ~ N(0,1); w_in [4c+cz, cz] and w_out [cz, c] ~ N(0, 1/fan_in) (standard deviation
    1/sqrt(fan_in)); dy [n,n,cz] ~ N(0,1); then gamma_in, gamma_out ~ 1 + 0.1 N(0,1) and beta_in, beta_out ~
    0.1 N(0,1), so that tests see the LayerNorm parameters act.  bf16 rounds every tensor (the oracle reads the
    rounded values).
    """
    g = torch.Generator().manual_seed(int(seed))
    z = torch.randn((n, n, cz), generator=g)
    w_in = torch.randn((4 * c + cz, cz), generator=g) / cz ** 0.5
    w_out = torch.randn((cz, c), generator=g) / c ** 0.5
    dy = torch.randn((n, n, cz), generator=g)
    gamma_in = 1.0 + 0.1 * torch.randn(cz, generator=g)
    beta_in = 0.1 * torch.randn(cz, generator=g)
    gamma_out = 1.0 + 0.1 * torch.randn(c, generator=g)
    beta_out = 0.1 * torch.randn(c, generator=g)
    out = dict(z=z, w_in=w_in, w_out=w_out, dy=dy, gamma_in=gamma_in, beta_in=beta_in, gamma_out=gamma_out,
               beta_out=beta_out)
    return {key: t.to(dtype) for key, t in out.items()}
