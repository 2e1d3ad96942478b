"""MI355X-native gated triangle self-attention with pair bias.

Thin ctypes binding over ``libtri_attn.so`` (see ``include/tri_attn.h``):
argument marshalling only, every step of the computation runs in the HIP
kernels.  PyTorch provides device memory and the stream.

    out, attn, lse = fwd(q, k, v, bias, gate, mask=None, ending=False)
    dq, dk, dv, dbias, dgate = bwd(q, k, v, bias, gate, mask, attn, lse, dout, ending=False)
    y, saved = block_fwd(z, gamma, beta, w_qkvg, w_bias, w_o, ending=False)   # LN + projections + attention + linear
    grads = block_bwd(z, gamma, beta, w_qkvg, w_bias, w_o, saved, dy, ending=False)

Layouts (starting node, N tokens, H heads, c = 32):
    q, k, v [N,H,N,c]; bias [H,N,N]; gate, out, dout [N,N,H,c]; mask [N,N] uint8
    (row i, key k; nonzero = keep) or None; attn [N,H,N,c]; lse [N,H,N] float32.
With ``ending=True`` the same tensors are taken in the caller's pair layout and
the operation runs around the ending node (the starting-node operation on the
transposed pair layout).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd", "bwd", "workspace_size", "bwd_chunk_rows", "fwd_workspace_size", "max_n", "TriAttnFunction",
           "tri_attn", "lib_path",
           "load", "ln_proj_fwd", "ln_proj_bwd", "out_proj_fwd", "out_proj_bwd", "block_fwd", "block_bwd",
           "block_fwd_chunked", "block_fwd_fused",
           "trimul_fwd", "trimul_bwd"]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libtri_attn.so")
_lib = None

F32, BF16 = 0, 1
_STATUS = {0: "ok", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP"}


def load():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with triangle_attention_tri_amd._build.build() "
                          "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(lib_path)
    i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.tri_attn_version.restype = i
    lib.tri_attn_status_string.argtypes = [i]
    lib.tri_attn_status_string.restype = ctypes.c_char_p
    lib.tri_attn_max_n.argtypes = [i]
    lib.tri_attn_max_n.restype = i
    lib.tri_attn_fwd_workspace_size.argtypes = [i, i, i, i, i]
    lib.tri_attn_fwd_workspace_size.restype = sz
    lib.tri_attn_fwd.argtypes = [i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tri_attn_fwd.restype = i
    lib.tri_attn_bwd_workspace_size.argtypes = [i, i, i, i, i]
    lib.tri_attn_bwd_workspace_size.restype = sz
    lib.tri_attn_bwd_chunk_rows.argtypes = [i, i, i, i, i]
    lib.tri_attn_bwd_chunk_rows.restype = i
    lib.tri_attn_bwd.argtypes = [i, i, i, i, i, i] + [vp] * 14 + [vp, sz, vp]
    lib.tri_attn_bwd.restype = i
    lib.tri_attn_fwd_noalloc.argtypes = [i, i, i, i, i, i] + [vp] * 9 + [vp]
    lib.tri_attn_fwd_noalloc.restype = i
    lib.tri_attn_fwd_noalloc_max_bytes.restype = sz
    lib.tri_attn_fwd_rc.argtypes = [i, i, i, i, i, i] + [vp] * 11 + [sz, vp]
    lib.tri_attn_fwd_rc.restype = i
    lib.tri_attn_bwd_rc.argtypes = [i, i, i, i, i, i] + [vp] * 15 + [vp, sz, vp]
    lib.tri_attn_bwd_rc.restype = i
    f = ctypes.c_float
    lib.tri_attn_ln_proj_fwd.argtypes = [i] * 6 + [vp, vp, vp, f] + [vp] * 9 + [vp]
    lib.tri_attn_ln_proj_fwd.restype = i
    lib.tri_attn_ln_proj_bwd_workspace_size.argtypes = [i] * 6
    lib.tri_attn_ln_proj_bwd_workspace_size.restype = sz
    lib.tri_attn_ln_proj_bwd.argtypes = [i] * 6 + [vp] * 17 + [vp, sz, vp]
    lib.tri_attn_ln_proj_bwd.restype = i
    lib.tri_attn_out_proj_fwd.argtypes = [i] * 4 + [vp] * 3 + [vp]
    lib.tri_attn_out_proj_fwd.restype = i
    lib.tri_attn_out_proj_bwd_workspace_size.argtypes = [i] * 4
    lib.tri_attn_out_proj_bwd_workspace_size.restype = sz
    lib.tri_attn_out_proj_bwd.argtypes = [i] * 4 + [vp] * 5 + [vp, sz, vp]
    lib.tri_attn_out_proj_bwd.restype = i
    lib.tri_attn_block_fwd_chunked_workspace_size.argtypes = [i] * 6
    lib.tri_attn_block_fwd_chunked_workspace_size.restype = sz
    lib.tri_attn_block_chunk_rows.argtypes = [i] * 5 + [sz]
    lib.tri_attn_block_chunk_rows.restype = i
    lib.tri_attn_block_fwd_chunked.argtypes = [i] * 6 + [vp, vp, vp, f, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tri_attn_block_fwd_chunked.restype = i
    lib.tri_attn_block_fwd_fused_workspace_size.argtypes = [i] * 6
    lib.tri_attn_block_fwd_fused_workspace_size.restype = sz
    lib.tri_attn_block_fwd_fused.argtypes = [i] * 6 + [vp, vp, vp, f, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tri_attn_block_fwd_fused.restype = i
    lib.tri_mul_saved_size.argtypes = [i] * 4
    lib.tri_mul_saved_size.restype = sz
    lib.tri_mul_workspace_size.argtypes = [i] * 4
    lib.tri_mul_workspace_size.restype = sz
    lib.tri_mul_fwd.argtypes = [i] * 5 + [vp] * 7 + [f, vp, vp, sz, vp]
    lib.tri_mul_fwd.restype = i
    lib.tri_mul_bwd.argtypes = [i] * 5 + [vp] * 7 + [f, vp, sz, vp] + [vp] * 7 + [vp, sz, vp]
    lib.tri_mul_bwd.restype = i
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        msg = load().tri_attn_status_string(status).decode()
        raise RuntimeError(f"{what} failed: {_STATUS.get(status, status)} ({msg})")


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dims(q, bias):
    n_rows, h, n, c = q.shape
    return n_rows, n, h, c


def _expect(name, t, shape):
    """Shape check before any library call: a smaller tensor would be read past its end."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _check_mask(mask, device, n_rows, n):
    import torch
    if mask is None:
        return
    if mask.dtype != torch.uint8 or mask.device != device or not mask.is_contiguous():
        raise TypeError("mask must be a contiguous uint8 tensor on the same device")
    _expect("mask", mask, (n_rows, n))


def _check_attention_shapes(q, k, v, bias, gate, n_rows, n, h, c, **more):
    """Layouts of the C ABI (both nodes: the ending node's tensors are the caller's full pair tensors, n_rows = n):
    q/k/v and attn [n_rows, h, n, c], bias [h, n, n], gate/out/dout [n_rows, n, h, c], lse [n_rows, h, n]."""
    shapes = dict(q=(n_rows, h, n, c), k=(n_rows, h, n, c), v=(n_rows, h, n, c), bias=(h, n, n),
                  gate=(n_rows, n, h, c), attn=(n_rows, h, n, c), attn_residual=(n_rows, h, n, c),
                  lse=(n_rows, h, n), dout=(n_rows, n, h, c))
    for name, t in dict(q=q, k=k, v=v, bias=bias, gate=gate, **more).items():
        _expect(name, t, shapes[name])


def _prep(tensors, dtype, device):
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def max_n(dtype) -> int:
    import torch
    return load().tri_attn_max_n(BF16 if dtype == torch.bfloat16 else F32)


def workspace_size(n_rows: int, n: int, h: int, c: int, dtype) -> int:
    """Backward workspace bytes."""
    import torch
    return int(load().tri_attn_bwd_workspace_size(n_rows, n, h, c, BF16 if dtype == torch.bfloat16 else F32))


def bwd_chunk_rows(n_rows: int, n: int, h: int, c: int, dtype) -> int:
    """Rows per chunk of the backward (it runs its rows in chunks that reuse one workspace)."""
    import torch
    return int(load().tri_attn_bwd_chunk_rows(n_rows, n, h, c, BF16 if dtype == torch.bfloat16 else F32))


def fwd_workspace_size(n_rows: int, n: int, h: int, c: int, dtype) -> int:
    import torch
    return int(load().tri_attn_fwd_workspace_size(n_rows, n, h, c, BF16 if dtype == torch.bfloat16 else F32))


def fwd(q, k, v, bias, gate, mask=None, ending: bool = False, workspace=None, residual: bool = False):
    """Forward.  Returns (out, attn, lse), or (out, attn, lse, attn_residual) with
    ``residual=True`` (bf16 only: int8 rounding-residual codes of attn, through
    tri_attn_fwd_rc)."""
    import torch
    lib = load()
    dt = _dtype_code(q)
    n_rows, n, h, c = _dims(q, bias)
    if ending:
        n_rows = n
    _prep(dict(q=q, k=k, v=v, bias=bias, gate=gate), q.dtype, q.device)
    _check_attention_shapes(q, k, v, bias, gate, n_rows, n, h, c)
    _check_mask(mask, q.device, n_rows, n)
    need = int(lib.tri_attn_fwd_workspace_size(n_rows, n, h, c, dt))
    if need == 0:
        _check(-2 if c != 32 else -1, "tri_attn_fwd_workspace_size")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = torch.empty_like(gate)
    attn = torch.empty((n_rows, h, n, c), dtype=q.dtype, device=q.device)
    lse = torch.empty((n_rows, h, n), dtype=torch.float32, device=q.device)
    if residual:
        res = torch.empty((n_rows, h, n, c), dtype=torch.int8, device=q.device)
        st = lib.tri_attn_fwd_rc(n_rows, n, h, c, dt, int(bool(ending)), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                 _ptr(gate), _ptr(mask), _ptr(out), _ptr(attn), _ptr(res), _ptr(lse),
                                 _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(q.device))
        _check(st, "tri_attn_fwd_rc")
        return out, attn, lse, res
    st = lib.tri_attn_fwd(n_rows, n, h, c, dt, int(bool(ending)), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                          _ptr(gate), _ptr(mask), _ptr(out), _ptr(attn), _ptr(lse), _ptr(workspace),
                          ctypes.c_size_t(workspace.numel()), _stream(q.device))
    _check(st, "tri_attn_fwd")
    return out, attn, lse


def bwd(q, k, v, bias, gate, mask, attn, lse, dout, ending: bool = False, workspace=None, attn_residual=None):
    """Backward.  Returns (dq, dk, dv, dbias, dgate).  ``attn_residual`` (the
    codes from ``fwd(..., residual=True)``) selects tri_attn_bwd_rc."""
    import torch
    lib = load()
    dt = _dtype_code(q)
    n_rows, n, h, c = _dims(q, bias)
    if ending:
        n_rows = n
    _prep(dict(q=q, k=k, v=v, bias=bias, gate=gate, attn=attn, dout=dout), q.dtype, q.device)
    _check_attention_shapes(q, k, v, bias, gate, n_rows, n, h, c, attn=attn, lse=lse, dout=dout,
                            attn_residual=attn_residual)
    _check_mask(mask, q.device, n_rows, n)
    if lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor on the same device")
    need = int(lib.tri_attn_bwd_workspace_size(n_rows, n, h, c, dt))
    if need == 0:
        _check(-2 if c != 32 else -1, "tri_attn_bwd_workspace_size")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbias, dgate = torch.empty_like(bias), torch.empty_like(gate)
    if attn_residual is not None:
        if attn_residual.dtype != torch.int8 or attn_residual.device != q.device or not attn_residual.is_contiguous():
            raise TypeError("attn_residual must be a contiguous int8 tensor on the same device")
        st = lib.tri_attn_bwd_rc(n_rows, n, h, c, dt, int(bool(ending)), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                 _ptr(gate), _ptr(mask), _ptr(attn), _ptr(attn_residual), _ptr(lse), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(dgate), _ptr(workspace),
                                 ctypes.c_size_t(workspace.numel()), _stream(q.device))
        _check(st, "tri_attn_bwd_rc")
        return dq, dk, dv, dbias, dgate
    st = lib.tri_attn_bwd(n_rows, n, h, c, dt, int(bool(ending)), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                          _ptr(gate), _ptr(mask), _ptr(attn), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(dbias), _ptr(dgate), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                          _stream(q.device))
    _check(st, "tri_attn_bwd")
    return dq, dk, dv, dbias, dgate


# ---------------------------------------------------------------------------
# LayerNorm + projection front end and output linear (bf16, c_z = h*c = 128)

def _check_front_shapes(cz, h, c, gamma, beta, w_qkvg, w_bias):
    _expect("gamma", gamma, (cz,))
    _expect("beta", beta, (cz,))
    _expect("w_qkvg", w_qkvg, (4 * h * c, cz))
    _expect("w_bias", w_bias, (h, cz))


def _check_out_shapes(o, w_o, dy=None):
    c_out, c_in = w_o.shape
    if o.dim() < 3 or o.shape[-2] * o.shape[-1] != c_in:
        raise ValueError(f"o must be [..., h, c] with h * c = {c_in}, got {list(o.shape)}")
    _expect("dy", dy, tuple(o.shape[:-2]) + (c_out,))


def ln_proj_fwd(z, gamma, beta, w_qkvg, w_bias, h: int = 4, c: int = 32, eps: float = 1e-5):
    """z [R,N,cz] -> (q, k, v [R,h,N,c], gate [R,N,h,c], bias [h,R,N], mean, rstd [R,N] fp32).

    For R < N (a slice of pair rows) ``bias`` is returned as [h,R,N]; the C ABI
    itself can also write into a full [h,N,N] tensor at a row offset.
    """
    import torch
    lib = load()
    n_rows, n, cz = z.shape
    _prep(dict(z=z, gamma=gamma, beta=beta, w_qkvg=w_qkvg, w_bias=w_bias), torch.bfloat16, z.device)
    _check_front_shapes(cz, h, c, gamma, beta, w_qkvg, w_bias)
    dev = z.device
    q = torch.empty((n_rows, h, n, c), dtype=z.dtype, device=dev)
    k, v = torch.empty_like(q), torch.empty_like(q)
    gate = torch.empty((n_rows, n, h, c), dtype=z.dtype, device=dev)
    bias = torch.empty((h, n_rows, n), dtype=z.dtype, device=dev) if n_rows == n else None
    mean = torch.empty((n_rows, n), dtype=torch.float32, device=dev)
    rstd = torch.empty_like(mean)
    if bias is None:
        raise ValueError("row slices: call the C ABI with the full bias tensor at a row offset")
    st = lib.tri_attn_ln_proj_fwd(n_rows, n, cz, h, c, BF16, _ptr(z), _ptr(gamma), _ptr(beta), ctypes.c_float(eps),
                                  _ptr(w_qkvg), _ptr(w_bias), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(bias),
                                  _ptr(mean), _ptr(rstd), _stream(dev))
    _check(st, "tri_attn_ln_proj_fwd")
    return q, k, v, gate, bias, mean, rstd


def ln_proj_bwd(z, gamma, beta, mean, rstd, w_qkvg, w_bias, dq, dk, dv, dgate, dbias, h: int = 4, c: int = 32,
                workspace=None):
    """Returns (dz, dgamma, dbeta, dw_qkvg, dw_bias)."""
    import torch
    lib = load()
    n_rows, n, cz = z.shape
    _prep(dict(z=z, gamma=gamma, beta=beta, w_qkvg=w_qkvg, w_bias=w_bias, dq=dq, dk=dk, dv=dv, dgate=dgate,
               dbias=dbias), torch.bfloat16, z.device)
    _check_front_shapes(cz, h, c, gamma, beta, w_qkvg, w_bias)
    if n_rows != n:
        raise ValueError("row slices: call the C ABI with the full dbias tensor at a row offset")
    for name, t in dict(dq=dq, dk=dk, dv=dv).items():
        _expect(name, t, (n_rows, h, n, c))
    _expect("dgate", dgate, (n_rows, n, h, c))
    _expect("dbias", dbias, (h, n, n))
    for name, t in dict(mean=mean, rstd=rstd).items():
        if t.dtype != torch.float32 or t.device != z.device or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous float32 tensor on the same device")
        _expect(name, t, (n_rows, n))
    need = int(lib.tri_attn_ln_proj_bwd_workspace_size(n_rows, n, cz, h, c, BF16))
    if need == 0:
        _check(-2, "tri_attn_ln_proj_bwd_workspace_size")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=z.device)
    dz = torch.empty_like(z)
    dgamma, dbeta = torch.empty_like(gamma), torch.empty_like(beta)
    dw_qkvg, dw_bias = torch.empty_like(w_qkvg), torch.empty_like(w_bias)
    st = lib.tri_attn_ln_proj_bwd(n_rows, n, cz, h, c, BF16, _ptr(z), _ptr(gamma), _ptr(beta), _ptr(mean),
                                  _ptr(rstd), _ptr(w_qkvg), _ptr(w_bias), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate),
                                  _ptr(dbias), _ptr(dz), _ptr(dgamma), _ptr(dbeta), _ptr(dw_qkvg), _ptr(dw_bias),
                                  _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(z.device))
    _check(st, "tri_attn_ln_proj_bwd")
    return dz, dgamma, dbeta, dw_qkvg, dw_bias


def out_proj_fwd(o, w_o):
    """o [..., h, c] (pairs first) -> y [..., c_out] = o.flatten(-2) @ w_o.T."""
    import torch
    lib = load()
    c_out, c_in = w_o.shape
    n_pairs = o.numel() // c_in
    _prep(dict(o=o, w_o=w_o), torch.bfloat16, o.device)
    _check_out_shapes(o, w_o)
    y = torch.empty(o.shape[:-2] + (c_out,), dtype=o.dtype, device=o.device)
    st = lib.tri_attn_out_proj_fwd(n_pairs, c_in, c_out, BF16, _ptr(o), _ptr(w_o), _ptr(y), _stream(o.device))
    _check(st, "tri_attn_out_proj_fwd")
    return y


def out_proj_bwd(o, w_o, dy, workspace=None):
    """Returns (do, dw_o)."""
    import torch
    lib = load()
    c_out, c_in = w_o.shape
    n_pairs = o.numel() // c_in
    _prep(dict(o=o, w_o=w_o, dy=dy), torch.bfloat16, o.device)
    _check_out_shapes(o, w_o, dy)
    need = int(lib.tri_attn_out_proj_bwd_workspace_size(n_pairs, c_in, c_out, BF16))
    if need == 0:
        _check(-2, "tri_attn_out_proj_bwd_workspace_size")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=o.device)
    d_o = torch.empty_like(o)
    dw_o = torch.empty_like(w_o)
    st = lib.tri_attn_out_proj_bwd(n_pairs, c_in, c_out, BF16, _ptr(o), _ptr(w_o), _ptr(dy), _ptr(d_o), _ptr(dw_o),
                                   _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(o.device))
    _check(st, "tri_attn_out_proj_bwd")
    return d_o, dw_o


def block_fwd(z, gamma, beta, w_qkvg, w_bias, w_o, ending: bool = False, mask=None, eps: float = 1e-5):
    """LayerNorm + projections -> attention (starting or ending node) -> output linear.

    Returns (y, saved) where ``saved`` holds what block_bwd needs.
    """
    q, k, v, gate, bias, mean, rstd = ln_proj_fwd(z, gamma, beta, w_qkvg, w_bias, eps=eps)
    out, attn, lse = fwd(q, k, v, bias, gate, mask, ending)
    y = out_proj_fwd(out, w_o)
    return y, dict(q=q, k=k, v=v, gate=gate, bias=bias, mean=mean, rstd=rstd, out=out, attn=attn, lse=lse)


def block_bwd(z, gamma, beta, w_qkvg, w_bias, w_o, saved, dy, ending: bool = False, mask=None):
    """Returns dict(dz, dgamma, dbeta, dw_qkvg, dw_bias, dw_o)."""
    s = saved
    d_out, dw_o = out_proj_bwd(s["out"], w_o, dy)
    dq, dk, dv, dbias, dgate = bwd(s["q"], s["k"], s["v"], s["bias"], s["gate"], mask, s["attn"], s["lse"], d_out,
                                   ending)
    dz, dgamma, dbeta, dw_qkvg, dw_bias = ln_proj_bwd(z, gamma, beta, s["mean"], s["rstd"], w_qkvg, w_bias, dq, dk,
                                                      dv, dgate, dbias)
    return dict(dz=dz, dgamma=dgamma, dbeta=dbeta, dw_qkvg=dw_qkvg, dw_bias=dw_bias, dw_o=dw_o)


def block_fwd_chunked(z, gamma, beta, w_qkvg, w_bias, w_o, mask=None, rows_per_chunk=None, budget_bytes=None,
                      eps: float = 1e-5, h: int = 4, c: int = 32):
    """Chunked inference of the starting-node block (tri_attn_block_fwd_chunked).

    ``rows_per_chunk`` pair rows at a time, or, with ``budget_bytes``, the
    largest chunk whose workspace fits (tri_attn_block_chunk_rows).  Returns
    (y, rows_per_chunk, workspace_bytes).
    """
    import torch
    lib = load()
    n, n2, cz = z.shape
    if n != n2:
        raise ValueError("z must be [n, n, c_z]")
    _prep(dict(z=z, gamma=gamma, beta=beta, w_qkvg=w_qkvg, w_bias=w_bias, w_o=w_o), torch.bfloat16, z.device)
    _check_mask(mask, z.device, n, n)
    if rows_per_chunk is None:
        if budget_bytes is None:
            raise ValueError("give rows_per_chunk or budget_bytes")
        rows_per_chunk = int(lib.tri_attn_block_chunk_rows(n, cz, h, c, BF16, ctypes.c_size_t(int(budget_bytes))))
        if rows_per_chunk == 0:
            raise ValueError("the budget does not hold even one pair row")
    need = int(lib.tri_attn_block_fwd_chunked_workspace_size(n, cz, h, c, BF16, int(rows_per_chunk)))
    if need == 0:
        _check(-1, "tri_attn_block_fwd_chunked_workspace_size")
    workspace = torch.empty(need, dtype=torch.uint8, device=z.device)
    y = torch.empty_like(z)
    st = lib.tri_attn_block_fwd_chunked(n, cz, h, c, BF16, int(rows_per_chunk), _ptr(z), _ptr(gamma), _ptr(beta),
                                        ctypes.c_float(eps), _ptr(w_qkvg), _ptr(w_bias), _ptr(w_o), _ptr(mask), _ptr(y),
                                        _ptr(workspace), ctypes.c_size_t(need), _stream(z.device))
    _check(st, "tri_attn_block_fwd_chunked")
    return y, int(rows_per_chunk), need


def block_fwd_fused(z, gamma, beta, w_qkvg, w_bias, w_o, mask=None, rows_per_chunk=None, eps: float = 1e-5,
                    h: int = 4, c: int = 32, workspace=None):
    """Fused inference of the starting-node block (tri_attn_block_fwd_fused): LayerNorm, q and the gate
    projected inside the attention kernel.  ``rows_per_chunk`` defaults to n.  Returns (y, workspace_bytes)."""
    import torch
    lib = load()
    n, n2, cz = z.shape
    if n != n2:
        raise ValueError("z must be [n, n, c_z]")
    _prep(dict(z=z, gamma=gamma, beta=beta, w_qkvg=w_qkvg, w_bias=w_bias, w_o=w_o), torch.bfloat16, z.device)
    _check_mask(mask, z.device, n, n)
    rows = n if rows_per_chunk is None else int(rows_per_chunk)
    need = int(lib.tri_attn_block_fwd_fused_workspace_size(n, cz, h, c, BF16, rows))
    if need == 0:
        _check(-1, "tri_attn_block_fwd_fused_workspace_size")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=z.device)
    y = torch.empty_like(z)
    st = lib.tri_attn_block_fwd_fused(n, cz, h, c, BF16, rows, _ptr(z), _ptr(gamma), _ptr(beta), ctypes.c_float(eps),
                                      _ptr(w_qkvg), _ptr(w_bias), _ptr(w_o), _ptr(mask), _ptr(y), _ptr(workspace),
                                      ctypes.c_size_t(need), _stream(z.device))
    _check(st, "tri_attn_block_fwd_fused")
    return y, need


# ---------------------------------------------------------------------------
# Triangular multiplicative update (include/tri_mul.h): bf16, c_z = c = 128

TRIMUL_PARAMS = ("gamma_in", "beta_in", "w_in", "gamma_out", "beta_out", "w_out")


def _trimul_check(z, p):
    import torch
    n, n2, cz = z.shape
    if n != n2:
        raise ValueError("z must be [n, n, c_z]")
    c = p["w_out"].shape[1]
    _prep(dict(z=z, **p), torch.bfloat16, z.device)
    for name, shape in dict(gamma_in=(cz,), beta_in=(cz,), w_in=(4 * c + cz, cz), gamma_out=(c,), beta_out=(c,),
                            w_out=(cz, c)).items():
        _expect(name, p[name], shape)
    return n, cz, c


def trimul_fwd(z, params: dict, incoming: bool = False, eps: float = 1e-5):
    """y = triangular multiplicative update of z [n, n, c_z] (outgoing or incoming edges).

    ``params`` holds gamma_in, beta_in, w_in [4c + c_z, c_z], gamma_out, beta_out, w_out [c_z, c].
    Returns (y, saved); ``saved`` is what trimul_bwd needs.
    """
    import torch
    lib = load()
    p = {k: params[k] for k in TRIMUL_PARAMS}
    n, cz, c = _trimul_check(z, p)
    need = int(lib.tri_mul_saved_size(n, cz, c, BF16))
    if need == 0:
        _check(-2, "tri_mul_saved_size")
    saved = torch.empty(need, dtype=torch.uint8, device=z.device)
    y = torch.empty_like(z)
    st = lib.tri_mul_fwd(n, cz, c, BF16, int(bool(incoming)), _ptr(z), *[_ptr(p[k]) for k in TRIMUL_PARAMS],
                         ctypes.c_float(eps), _ptr(y), _ptr(saved), ctypes.c_size_t(need), _stream(z.device))
    _check(st, "tri_mul_fwd")
    return y, saved


def trimul_bwd(z, params: dict, saved, dy, incoming: bool = False, eps: float = 1e-5, workspace=None):
    """Returns dict(dz, dgamma_in, dbeta_in, dw_in, dgamma_out, dbeta_out, dw_out)."""
    import torch
    lib = load()
    p = {k: params[k] for k in TRIMUL_PARAMS}
    n, cz, c = _trimul_check(z, p)
    _prep(dict(dy=dy), torch.bfloat16, z.device)
    _expect("dy", dy, tuple(z.shape))
    need = int(lib.tri_mul_workspace_size(n, cz, c, BF16))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=z.device)
    out = dict(dz=torch.empty_like(z), **{"d" + k: torch.empty_like(p[k]) for k in TRIMUL_PARAMS})
    st = lib.tri_mul_bwd(n, cz, c, BF16, int(bool(incoming)), _ptr(z), *[_ptr(p[k]) for k in TRIMUL_PARAMS],
                         ctypes.c_float(eps), _ptr(saved), ctypes.c_size_t(saved.numel()), _ptr(dy), _ptr(out["dz"]),
                         *[_ptr(out["d" + k]) for k in TRIMUL_PARAMS], _ptr(workspace),
                         ctypes.c_size_t(workspace.numel()), _stream(z.device))
    _check(st, "tri_mul_bwd")
    return out


def __getattr__(name):
    if name in ("TriAttnFunction", "tri_attn"):
        from . import autograd as _ag
        return getattr(_ag, name)
    raise AttributeError(name)
