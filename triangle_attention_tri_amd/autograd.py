"""torch.autograd wrapper over the C ABI (forward saves attn and lse)."""
from __future__ import annotations

import torch

from . import bwd as _bwd
from . import fwd as _fwd


class TriAttnFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, bias, gate, mask=None, ending=False):
        out, attn, lse = _fwd(q, k, v, bias, gate, mask, ending)
        ctx.save_for_backward(q, k, v, bias, gate, attn, lse)
        ctx.mask = mask
        ctx.ending = ending
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, bias, gate, attn, lse = ctx.saved_tensors
        dq, dk, dv, dbias, dgate = _bwd(q, k, v, bias, gate, ctx.mask, attn, lse, dout.contiguous(), ctx.ending)
        return dq, dk, dv, dbias, dgate, None, None


def tri_attn(q, k, v, bias, gate, mask=None, ending=False):
    return TriAttnFunction.apply(q, k, v, bias, gate, mask, ending)
