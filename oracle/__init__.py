"""fp64 CPU oracle for gated triangle self-attention with pair bias.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``triangle_attention_tri_amd``) and never imports it.

The attention itself is plain C (``tri_oracle.c``, fp64, one thread per
(row, head) task); this module only converts arrays to contiguous float64,
calls it, and composes the ending node and the LayerNorm / projection block
from the starting node with plain numpy.

Sources for what is computed (the pages state it in words only):
* TurboPairFormer news item (ai.info), section "Dove si impiega il tempo":
  attention of a pair over a third token, cubic cost, backward yields
  gradients of query, key, value and pair bias.
* HelixFold review (nubint.ai), "Fused Gated Self-Attention": the attention is
  gated.
* MegaFold explainer (gist.science), EvoFlash-3D paragraph: the N^2 x N map of
  pair-to-third-token interactions.
The exact formula, layouts and the ending-node definition follow the
configuration statements of this workload (starting node
o_ij = sigmoid(g_ij) * sum_k softmax_k(q_ij . k_ik / sqrt(c) + b_jk) v_ik;
ending node = the same operation on the transposed pair layout).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tri_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtri_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-shared", "-fPIC", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i = ctypes.c_int
        lib.oracle_fwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, u8p, dp, dp, dp, i]
        lib.oracle_fwd.restype = i
        lib.oracle_bwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, u8p, dp,
                                   dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_bwd.restype = i
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Widen to contiguous float64 (exact for float32 and bfloat16-valued data)."""
    if hasattr(x, "detach"):  # torch tensor: bf16 -> f32 is exact, then f64
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _u8(m):
    if m is None:
        return None
    if hasattr(m, "detach"):
        m = m.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(m) != 0, dtype=np.uint8)


def _ptr(a, ty=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ty))


def _shapes(q, k, bias, gate, mask):
    rows, H, nq, c = q.shape
    assert k.shape[0] == rows and k.shape[1] == H and k.shape[3] == c, "k shape"
    nk = k.shape[2]
    assert bias.shape == (H, nq, nk), f"bias shape {bias.shape} != {(H, nq, nk)}"
    assert gate.shape == (rows, nq, H, c), "gate shape"
    if mask is not None:
        assert mask.shape == (rows, nk), "mask shape"
    return rows, H, nq, nk, c


def attn_fwd(q, k, v, bias, gate, mask=None, threads: int = 0):
    """Starting-node forward.

    q [rows,H,nq,c]; k, v [rows,H,nk,c]; bias [H,nq,nk]; gate [rows,nq,H,c];
    mask [rows,nk] (nonzero = keep) or None.
    Returns dict(out [rows,nq,H,c], attn [rows,H,nq,c], lse [rows,H,nq], threads).
    """
    q, k, v, bias, gate = (_f64(t) for t in (q, k, v, bias, gate))
    mask = _u8(mask)
    rows, H, nq, nk, c = _shapes(q, k, bias, gate, mask)
    out = np.zeros((rows, nq, H, c))
    attn = np.zeros((rows, H, nq, c))
    lse = np.zeros((rows, H, nq))
    used = _load().oracle_fwd(rows, H, nq, nk, c, _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(gate),
                              _ptr(mask, ctypes.c_uint8), _ptr(out), _ptr(attn), _ptr(lse), threads)
    return dict(out=out, attn=attn, lse=lse, threads=used)


def attn_bwd(q, k, v, bias, gate, mask, dout, threads: int = 0):
    """Starting-node forward + backward.

    Returns dict(out, attn, lse, dq, dk, dv, dbias [H,nq,nk] summed over the
    rows given, dgate, D [rows,H,nq], d_mismatch, threads).
    """
    q, k, v, bias, gate, dout = (_f64(t) for t in (q, k, v, bias, gate, dout))
    mask = _u8(mask)
    rows, H, nq, nk, c = _shapes(q, k, bias, gate, mask)
    assert dout.shape == gate.shape, "dout shape"
    r = dict(out=np.zeros((rows, nq, H, c)), attn=np.zeros((rows, H, nq, c)), lse=np.zeros((rows, H, nq)),
             dq=np.zeros((rows, H, nq, c)), dk=np.zeros((rows, H, nk, c)), dv=np.zeros((rows, H, nk, c)),
             dbias=np.zeros((H, nq, nk)), dgate=np.zeros((rows, nq, H, c)), D=np.zeros((rows, H, nq)))
    mis = ctypes.c_double(0.0)
    used = _load().oracle_bwd(rows, H, nq, nk, c, _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(gate),
                              _ptr(mask, ctypes.c_uint8), _ptr(dout),
                              _ptr(r["out"]), _ptr(r["attn"]), _ptr(r["lse"]),
                              _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dbias"]),
                              _ptr(r["dgate"]), _ptr(r["D"]), ctypes.byref(mis), threads)
    r["d_mismatch"] = mis.value
    r["threads"] = used
    return r


# ---------------------------------------------------------------------------
# Ending node: the same operation on the transposed pair layout.  T swaps the
# two pair axes of every pair-indexed tensor; end = T o start o T.

def _t_qkv(x):      # [a,H,b,c] -> [b,H,a,c]
    return np.ascontiguousarray(np.transpose(x, (2, 1, 0, 3)))


def _t_pair(x):     # [a,b,H,c] -> [b,a,H,c]
    return np.ascontiguousarray(np.transpose(x, (1, 0, 2, 3)))


def _t_bias(x):     # [H,a,b] -> [H,b,a]
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1)))


def _t_mask(m):     # [a,b] -> [b,a]
    return None if m is None else np.ascontiguousarray(np.transpose(m))


def attn_end_fwd(q, k, v, bias, gate, mask=None, threads: int = 0):
    """Ending-node forward on tensors held in the pair layout (square N x N).

    Returned ``out`` is in the caller's pair layout; ``attn`` and ``lse`` are in
    the transposed (kernel) order [i,H,j,...] of the starting-node call.
    """
    q, k, v, bias, gate = (_f64(t) for t in (q, k, v, bias, gate))
    mask = _u8(mask)
    r = attn_fwd(_t_qkv(q), _t_qkv(k), _t_qkv(v), _t_bias(bias), _t_pair(gate), _t_mask(mask), threads)
    r["out"] = _t_pair(r["out"])
    return r


def attn_end_bwd(q, k, v, bias, gate, mask, dout, threads: int = 0):
    q, k, v, bias, gate, dout = (_f64(t) for t in (q, k, v, bias, gate, dout))
    mask = _u8(mask)
    r = attn_bwd(_t_qkv(q), _t_qkv(k), _t_qkv(v), _t_bias(bias), _t_pair(gate), _t_mask(mask),
                 _t_pair(dout), threads)
    r["out"] = _t_pair(r["out"])
    for key in ("dq", "dk", "dv"):
        r[key] = _t_qkv(r[key])
    r["dgate"] = _t_pair(r["dgate"])
    r["dbias"] = _t_bias(r["dbias"])
    return r
