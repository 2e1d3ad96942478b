"""C ABI contract, checked on the CPU (no kernel is launched).

* libtri_attn.so loads and exports every function declared in include/tri_attn.h.
* Argument validation returns the documented negative status before any HIP
  call, so these calls are safe without a GPU.
* Workspace sizes are consistent with the documented bounds.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import triangle_attention_tri_amd as ta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tri_attn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(tri_(?:attn|mul)_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ta.lib_path):
        from triangle_attention_tri_amd import _build
        _build.build()
    return ta.load()


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert {"tri_attn_fwd", "tri_attn_bwd", "tri_attn_bwd_workspace_size", "tri_mul_fwd", "tri_mul_bwd"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in tri_attn.h but not exported"


def test_status_strings(lib):
    for st in (OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, 12345):
        s = lib.tri_attn_status_string(st)
        assert isinstance(s, bytes) and len(s) > 0


def test_version_and_limits(lib):
    assert lib.tri_attn_version() >= 100
    assert lib.tri_attn_max_n(ta.BF16) >= 768
    assert lib.tri_attn_max_n(ta.F32) >= 256
    assert lib.tri_attn_max_n(7) == 0


def fake_ptr(offset=0):
    # aligned, non-null, never dereferenced: validation rejects the call first
    return ctypes.c_void_p(0x10000 + offset)


def call_fwd(lib, n_rows=8, n=8, h=2, c=32, dtype=ta.BF16, ending=0, ptrs=None, ws_bytes=None, ws=None):
    p = ptrs or [fake_ptr()] * 8
    if ws_bytes is None:
        ws_bytes = lib.tri_attn_fwd_workspace_size(n_rows, n, h, 32, dtype)
    ws = fake_ptr(0x100000) if ws is None else ws
    return lib.tri_attn_fwd(n_rows, n, h, c, dtype, ending, p[0], p[1], p[2], p[3], p[4], None, p[5], p[6], p[7],
                            ws, ctypes.c_size_t(ws_bytes), None)


def call_bwd(lib, n_rows=8, n=8, h=2, c=32, dtype=ta.BF16, ending=0, ptrs=None, ws_bytes=None, ws=None):
    p = ptrs or [fake_ptr()] * 13
    if ws_bytes is None:
        ws_bytes = lib.tri_attn_bwd_workspace_size(n_rows, n, h, 32, dtype)
    ws = fake_ptr(0x100000) if ws is None else ws
    return lib.tri_attn_bwd(n_rows, n, h, c, dtype, ending, p[0], p[1], p[2], p[3], p[4], None, p[5], p[6], p[7],
                            p[8], p[9], p[10], p[11], p[12], ws, ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("call", [call_fwd, call_bwd])
def test_validation_errors(lib, call):
    assert call(lib, n_rows=0) == EINVAL
    assert call(lib, n=0) == EINVAL
    assert call(lib, h=0) == EINVAL
    assert call(lib, n_rows=9, n=8) == EINVAL          # more rows than the pair axis holds
    assert call(lib, dtype=5) == EINVAL
    assert call(lib, ending=2) == EINVAL
    assert call(lib, c=16) == EUNSUPPORTED
    assert call(lib, c=64) == EUNSUPPORTED
    big = lib.tri_attn_max_n(ta.BF16) + 1
    assert call(lib, n_rows=1, n=big, ws_bytes=1 << 40) == EUNSUPPORTED


@pytest.mark.parametrize("call,nptr", [(call_fwd, 8), (call_bwd, 13)])
def test_null_and_misaligned(lib, call, nptr):
    for i in range(nptr):
        ptrs = [fake_ptr()] * nptr
        ptrs[i] = None
        assert call(lib, ptrs=ptrs) == EINVAL, f"null pointer {i}"
        ptrs[i] = fake_ptr(2)
        assert call(lib, ptrs=ptrs) == EINVAL, f"misaligned pointer {i}"


@pytest.mark.parametrize("call", [call_fwd, call_bwd])
def test_workspace_errors(lib, call):
    assert call(lib, ws=ctypes.c_void_p(0)) == EWORKSPACE
    need = (lib.tri_attn_fwd_workspace_size if call is call_fwd else lib.tri_attn_bwd_workspace_size)(8, 8, 2, 32,
                                                                                                       ta.BF16)
    assert need > 0
    assert call(lib, ws_bytes=need - 1) == EWORKSPACE
    assert call(lib, ws=fake_ptr(0x100000 + 16)) == EINVAL   # workspace must be 256-byte aligned


def test_workspace_sizes(lib):
    for dt in (ta.BF16, ta.F32):
        assert lib.tri_attn_bwd_workspace_size(8, 8, 2, 16, dt) == 0
        assert lib.tri_attn_fwd_workspace_size(0, 8, 2, 32, dt) == 0
        prev = 0
        for n in (1, 17, 64, 127, 256):
            b = lib.tri_attn_bwd_workspace_size(n, n, 4, 32, dt)
            f = lib.tri_attn_fwd_workspace_size(n, n, 4, 32, dt)
            assert b % 256 == 0 and f % 256 == 0
            assert b > prev
            prev = b
            # at least the gradient reaching the pre-gate attention and the per-query D
            assert b >= n * 4 * n * 32 * (2 if dt == ta.BF16 else 4) + n * 4 * n * 4


def test_backward_chunks(lib):
    """The backward runs its rows in chunks that bound the workspace: one chunk for small calls, whole 32-row
    blocks otherwise, and at N=768, H=4 (bf16) a workspace under 0.6 GB (a single pass would need 1.9 GB)."""
    lib.tri_attn_bwd_chunk_rows.argtypes = [ctypes.c_int] * 5
    assert lib.tri_attn_bwd_chunk_rows(8, 8, 2, 16, ta.BF16) == 0
    assert lib.tri_attn_bwd_chunk_rows(0, 8, 2, 32, ta.BF16) == 0
    for dt in (ta.BF16, ta.F32):
        for n in (1, 17, 64, 256):
            assert lib.tri_attn_bwd_chunk_rows(n, n, 4, 32, dt) == n
    for n, dt in ((640, ta.BF16), (768, ta.BF16), (960, ta.BF16), (2048, ta.BF16), (300, ta.F32), (736, ta.F32)):
        ch = lib.tri_attn_bwd_chunk_rows(n, n, 4, 32, dt)
        assert 32 <= ch <= n and (ch == n or ch % 32 == 0), (n, dt, ch)
        # a row slice never gets a larger chunk than the full call
        assert lib.tri_attn_bwd_chunk_rows(n // 2, n, 4, 32, dt) == min(ch, n // 2)
    assert lib.tri_attn_bwd_chunk_rows(768, 768, 4, 32, ta.BF16) < 768
    assert lib.tri_attn_bwd_workspace_size(768, 768, 4, 32, ta.BF16) <= 600_000_000
    # beyond the input-sized dA and D of every row: one chunk of at least 32 rows of partial sums, the prepared
    # bias tiles and the running pair-bias sum
    n = 2048
    assert lib.tri_attn_bwd_workspace_size(n, n, 4, 32, ta.BF16) <= n * 4 * n * (32 * 2 + 4) + 700_000_000


def test_noalloc_forward_limits(lib):
    """tri_attn_fwd_noalloc rejects, before any device call, sizes whose scratch exceeds its fixed array and the
    forward's usual argument errors."""
    assert lib.tri_attn_fwd_noalloc_max_bytes() == 16 << 20
    p = fake_ptr(0x100000)
    args = lambda n, dt=ta.BF16, c=32, ptr=p: (n, n, 4, c, dt, 0, ptr, ptr, ptr, ptr, ptr, None, ptr, ptr, ptr,  # noqa
                                               None)
    assert lib.tri_attn_fwd_noalloc(*args(1100)) == EWORKSPACE      # h * ceil(n/32)^2 * 4 KiB > 16 MiB
    assert lib.tri_attn_fwd_noalloc(*args(64, c=16)) == EUNSUPPORTED
    assert lib.tri_attn_fwd_noalloc(*args(64, dt=7)) == EINVAL
    assert lib.tri_attn_fwd_noalloc(*args(64, ptr=fake_ptr(0x100008))) == EINVAL


def test_binding_rejects_bad_inputs():
    q = torch.zeros((4, 2, 4, 32), dtype=torch.float16)
    with pytest.raises(TypeError):
        ta.fwd(q, q, q, torch.zeros((2, 4, 4), dtype=torch.float16), torch.zeros((4, 4, 2, 32), dtype=torch.float16))


# --- the block entry points (front end, output linear) ----------------------------------
def call_ln_proj_fwd(lib, n_rows=8, n=8, cz=128, h=4, c=32, dtype=ta.BF16, eps=1e-5, ptrs=None):
    p = ptrs or [fake_ptr()] * 12
    return lib.tri_attn_ln_proj_fwd(n_rows, n, cz, h, c, dtype, p[0], p[1], p[2], ctypes.c_float(eps), p[3], p[4],
                                    p[5], p[6], p[7], p[8], p[9], p[10], p[11], None)


def call_ln_proj_bwd(lib, n_rows=8, n=8, cz=128, h=4, c=32, dtype=ta.BF16, ptrs=None, ws_bytes=None, ws=None):
    p = ptrs or [fake_ptr()] * 17
    if ws_bytes is None:
        ws_bytes = lib.tri_attn_ln_proj_bwd_workspace_size(n_rows, n, cz, h, c, dtype)
    ws = fake_ptr(0x100000) if ws is None else ws
    return lib.tri_attn_ln_proj_bwd(n_rows, n, cz, h, c, dtype, *p, ws, ctypes.c_size_t(ws_bytes), None)


def call_out_proj_bwd(lib, n_pairs=64, c_in=128, c_out=128, dtype=ta.BF16, ptrs=None, ws_bytes=None, ws=None):
    p = ptrs or [fake_ptr()] * 5
    if ws_bytes is None:
        ws_bytes = lib.tri_attn_out_proj_bwd_workspace_size(n_pairs, c_in, c_out, dtype)
    ws = fake_ptr(0x100000) if ws is None else ws
    return lib.tri_attn_out_proj_bwd(n_pairs, c_in, c_out, dtype, *p, ws, ctypes.c_size_t(ws_bytes), None)


def test_block_validation(lib):
    assert call_ln_proj_fwd(lib, n_rows=0) == EINVAL
    assert call_ln_proj_fwd(lib, n_rows=9, n=8) == EINVAL
    assert call_ln_proj_fwd(lib, dtype=3) == EINVAL
    assert call_ln_proj_fwd(lib, dtype=ta.F32) == EUNSUPPORTED       # bf16 only
    assert call_ln_proj_fwd(lib, cz=64) == EUNSUPPORTED
    assert call_ln_proj_fwd(lib, h=2) == EUNSUPPORTED                # h*c must be 128
    assert call_ln_proj_fwd(lib, eps=0.0) == EINVAL
    for i in range(12):
        ptrs = [fake_ptr()] * 12
        ptrs[i] = None
        assert call_ln_proj_fwd(lib, ptrs=ptrs) == EINVAL, f"null pointer {i}"
    assert call_ln_proj_bwd(lib, cz=64) == EUNSUPPORTED
    assert call_ln_proj_bwd(lib, ws=ctypes.c_void_p(0)) == EWORKSPACE
    need = lib.tri_attn_ln_proj_bwd_workspace_size(8, 8, 128, 4, 32, ta.BF16)
    assert need > 0 and need % 256 == 0
    assert call_ln_proj_bwd(lib, ws_bytes=need - 1) == EWORKSPACE
    assert call_ln_proj_bwd(lib, ws=fake_ptr(0x100000 + 16)) == EINVAL
    assert lib.tri_attn_out_proj_fwd(64, 128, 64, ta.BF16, fake_ptr(), fake_ptr(), fake_ptr(), None) == EUNSUPPORTED
    assert lib.tri_attn_out_proj_fwd(0, 128, 128, ta.BF16, fake_ptr(), fake_ptr(), fake_ptr(), None) == EINVAL
    assert lib.tri_attn_out_proj_fwd(64, 128, 128, ta.BF16, fake_ptr(2), fake_ptr(), fake_ptr(), None) == EINVAL
    assert call_out_proj_bwd(lib, c_out=64) == EUNSUPPORTED
    assert call_out_proj_bwd(lib, ws=ctypes.c_void_p(0)) == EWORKSPACE
    assert lib.tri_attn_out_proj_bwd_workspace_size(64, 128, 128, ta.BF16) > 0
    assert lib.tri_attn_ln_proj_bwd_workspace_size(8, 8, 128, 4, 32, ta.F32) == 0


def call_fwd_rc(lib, dtype=ta.BF16, res=None, n_rows=8, ptrs=None):
    p = ptrs or [fake_ptr()] * 8
    ws_bytes = lib.tri_attn_fwd_workspace_size(8, 8, 2, 32, ta.BF16)
    return lib.tri_attn_fwd_rc(n_rows, 8, 2, 32, dtype, 0, p[0], p[1], p[2], p[3], p[4], None, p[5], p[6], res, p[7],
                               fake_ptr(0x100000), ctypes.c_size_t(ws_bytes), None)


def call_bwd_rc(lib, dtype=ta.BF16, res=None, n_rows=8, ptrs=None):
    p = ptrs or [fake_ptr()] * 13
    ws_bytes = lib.tri_attn_bwd_workspace_size(8, 8, 2, 32, ta.BF16)
    return lib.tri_attn_bwd_rc(n_rows, 8, 2, 32, dtype, 0, p[0], p[1], p[2], p[3], p[4], None, p[5], res, p[6],
                               p[7], p[8], p[9], p[10], p[11], p[12], fake_ptr(0x100000), ctypes.c_size_t(ws_bytes),
                               None)


@pytest.mark.parametrize("call,nptr", [(call_fwd_rc, 8), (call_bwd_rc, 13)])
def test_residual_entry_validation(lib, call, nptr):
    """The residual-compensated pair: bf16 only, residual buffer required and 16-byte aligned; the other
    arguments are checked as for tri_attn_fwd / tri_attn_bwd (no call here reaches a launch)."""
    good = fake_ptr(0x200000)
    assert call(lib, dtype=ta.F32, res=good) == EINVAL
    assert call(lib, res=None) == EINVAL
    assert call(lib, res=fake_ptr(0x200000 + 8)) == EINVAL
    assert call(lib, res=good, n_rows=0) == EINVAL
    for i in range(nptr):
        ptrs = [fake_ptr()] * nptr
        ptrs[i] = None
        assert call(lib, res=good, ptrs=ptrs) == EINVAL, f"null pointer {i}"


def test_chunked_block_contract(lib):
    """Workspace sizes and the budget -> chunk choice of the chunked block forward, and its argument checks
    (none of these calls reaches a launch)."""
    n, cz, h, c = 64, 128, 4, 32
    size = lambda r: lib.tri_attn_block_fwd_chunked_workspace_size(n, cz, h, c, ta.BF16, r)  # noqa: E731
    sizes = [size(r) for r in range(1, n + 1)]
    assert all(s > 0 and s % 256 == 0 for s in sizes)
    assert all(a < b for a, b in zip(sizes, sizes[1:]))
    assert size(0) == 0 and size(n + 1) == 0
    assert lib.tri_attn_block_fwd_chunked_workspace_size(n, cz, h, c, ta.F32, 8) == 0
    assert lib.tri_attn_block_fwd_chunked_workspace_size(n, 64, h, c, ta.BF16, 8) == 0
    # at least the full bias and one row of the four projections
    assert sizes[0] >= h * n * n * 2 + 4 * n * h * c * 2
    for r in (1, 7, 32, n):
        assert lib.tri_attn_block_chunk_rows(n, cz, h, c, ta.BF16, ctypes.c_size_t(size(r))) == r
        assert lib.tri_attn_block_chunk_rows(n, cz, h, c, ta.BF16, ctypes.c_size_t(size(r) + 255)) == r
    assert lib.tri_attn_block_chunk_rows(n, cz, h, c, ta.BF16, ctypes.c_size_t(size(1) - 1)) == 0
    assert lib.tri_attn_block_chunk_rows(n, cz, h, c, ta.BF16, ctypes.c_size_t(1 << 40)) == n

    def call(rows=8, y=fake_ptr(), ws_bytes=None, eps=1e-5):
        need = size(8) if ws_bytes is None else ws_bytes
        return lib.tri_attn_block_fwd_chunked(n, cz, h, c, ta.BF16, rows, fake_ptr(), fake_ptr(), fake_ptr(),
                                              ctypes.c_float(eps), fake_ptr(), fake_ptr(), fake_ptr(), None, y,
                                              fake_ptr(0x100000), ctypes.c_size_t(need), None)
    assert call(rows=0) == EINVAL
    assert call(rows=n + 1) == EINVAL
    assert call(y=None) == EINVAL
    assert call(y=fake_ptr(2)) == EINVAL
    assert call(eps=0.0) == EINVAL
    assert call(ws_bytes=size(8) - 1) == EWORKSPACE


def test_chunked_binding_rejects_mask_shape():
    """The binding checks the mask's shape before any call into the library (a smaller mask would be
    read past its end)."""
    import torch
    n, cz = 8, 128
    bf = dict(dtype=torch.bfloat16)
    z = torch.zeros(n, n, cz, **bf)
    args = (z, torch.ones(cz, **bf), torch.zeros(cz, **bf), torch.zeros(512, cz, **bf), torch.zeros(4, cz, **bf),
            torch.zeros(cz, 128, **bf))
    with pytest.raises(ValueError, match="mask must have shape"):
        ta.block_fwd_chunked(*args, mask=torch.ones(n, n - 1, dtype=torch.uint8), rows_per_chunk=4)


def test_attention_binding_shape_checks():
    """fwd / bwd reject tensors whose shapes do not match the layouts of the C ABI, before any call into the
    library (the kernels would read past the end of a smaller tensor)."""
    import torch
    n_rows, n, h, c = 3, 8, 4, 32
    bf = dict(dtype=torch.bfloat16)
    q = torch.zeros(n_rows, h, n, c, **bf)
    bias = torch.zeros(h, n, n, **bf)
    gate = torch.zeros(n_rows, n, h, c, **bf)
    lse = torch.zeros(n_rows, h, n)
    with pytest.raises(ValueError, match="gate must have shape"):
        ta.fwd(q, q, q, bias, torch.zeros(n_rows, n - 1, h, c, **bf))
    with pytest.raises(ValueError, match="k must have shape"):
        ta.fwd(q, q[:, :, :-1].contiguous(), q, bias, gate)
    with pytest.raises(ValueError, match="bias must have shape"):
        ta.fwd(q, q, q, torch.zeros(h, n, n - 1, **bf), gate)
    with pytest.raises(ValueError, match="mask must have shape"):
        ta.fwd(q, q, q, bias, gate, torch.ones(n, n, dtype=torch.uint8))  # n_rows < n: one row per processed row
    with pytest.raises(ValueError, match="q must have shape"):
        ta.fwd(q, q, q, bias, gate, ending=True)  # the ending node takes the full [n, h, n, c] tensors
    with pytest.raises(ValueError, match="lse must have shape"):
        ta.bwd(q, q, q, bias, gate, None, q, lse[:, :, :-1].contiguous(), gate)
    with pytest.raises(TypeError, match="lse must be"):
        ta.bwd(q, q, q, bias, gate, None, q, lse.to(torch.float64), gate)
    with pytest.raises(TypeError, match="mask must be"):
        ta.bwd(q, q, q, bias, gate, torch.ones(n_rows, n, dtype=torch.int32), q, lse, gate)
    with pytest.raises(ValueError, match="attn_residual must have shape"):
        ta.bwd(q, q, q, bias, gate, None, q, lse, gate, attn_residual=torch.zeros(1, h, n, c, dtype=torch.int8))


def test_projection_binding_shape_checks():
    """The front-end and output-linear bindings check weight, statistics and gradient shapes before any call
    into the library."""
    import torch
    n, cz, h, c = 8, 128, 4, 32
    bf = dict(dtype=torch.bfloat16)
    z = torch.zeros(n, n, cz, **bf)
    g, b = torch.ones(cz, **bf), torch.zeros(cz, **bf)
    w, wb = torch.zeros(4 * h * c, cz, **bf), torch.zeros(h, cz, **bf)
    with pytest.raises(ValueError, match="w_qkvg must have shape"):
        ta.ln_proj_fwd(z, g, b, w[:-1].contiguous(), wb)
    with pytest.raises(ValueError, match="gamma must have shape"):
        ta.ln_proj_fwd(z, g[:-1].contiguous(), b, w, wb)
    dqkv = torch.zeros(n, h, n, c, **bf)
    dgate = torch.zeros(n, n, h, c, **bf)
    stat = torch.zeros(n, n)
    with pytest.raises(ValueError, match="dbias must have shape"):
        ta.ln_proj_bwd(z, g, b, stat, stat, w, wb, dqkv, dqkv, dqkv, dgate, torch.zeros(h, n, n - 1, **bf))
    with pytest.raises(TypeError, match="mean must be"):
        ta.ln_proj_bwd(z, g, b, stat.bfloat16(), stat, w, wb, dqkv, dqkv, dqkv, dgate, torch.zeros(h, n, n, **bf))
    w_o = torch.zeros(cz, h * c, **bf)
    with pytest.raises(ValueError, match="o must be"):
        ta.out_proj_fwd(torch.zeros(n, n, h, c - 1, **bf), w_o)
    with pytest.raises(ValueError, match="dy must have shape"):
        ta.out_proj_bwd(torch.zeros(n, n, h, c, **bf), w_o, torch.zeros(n, n - 1, cz, **bf))


def test_trimul_validation(lib):
    """tri_mul_* reject bad arguments before any device call."""
    p = fake_ptr(0x100000)
    big = ctypes.c_size_t(1 << 40)
    f = ctypes.c_float

    def fwd(n=64, cz=128, c=128, dt=ta.BF16, inc=0, ptr=p, eps=1e-5, saved=p, saved_bytes=big):
        return lib.tri_mul_fwd(n, cz, c, dt, inc, ptr, p, p, p, p, p, p, f(eps), p, saved, saved_bytes, None)

    def bwd(n=64, ws=p, ws_bytes=big, saved_bytes=big, ptr=p):
        return lib.tri_mul_bwd(n, 128, 128, ta.BF16, 0, ptr, p, p, p, p, p, p, f(1e-5), p, saved_bytes, p,
                               p, p, p, p, p, p, p, ws, ws_bytes, None)
    assert lib.tri_mul_saved_size(64, 128, 128, ta.BF16) > 0 and lib.tri_mul_workspace_size(64, 128, 128, ta.BF16) > 0
    assert lib.tri_mul_saved_size(64, 64, 128, ta.BF16) == 0 and lib.tri_mul_saved_size(0, 128, 128, ta.BF16) == 0
    assert fwd(n=0) == EINVAL and fwd(inc=2) == EINVAL and fwd(dt=5) == EINVAL
    assert fwd(cz=64) == EUNSUPPORTED and fwd(c=96) == EUNSUPPORTED and fwd(dt=ta.F32) == EUNSUPPORTED
    assert fwd(n=5000) == EUNSUPPORTED
    assert fwd(eps=0.0) == EINVAL and fwd(ptr=fake_ptr(0x100008)) == EINVAL and fwd(ptr=None) == EINVAL
    assert fwd(saved=None) == EWORKSPACE and fwd(saved_bytes=ctypes.c_size_t(100)) == EWORKSPACE
    assert fwd(saved=fake_ptr(0x100000 + 16)) == EINVAL
    assert bwd(ws=None) == EWORKSPACE and bwd(saved_bytes=ctypes.c_size_t(10)) == EWORKSPACE
    assert bwd(ptr=fake_ptr(0x100004)) == EINVAL
