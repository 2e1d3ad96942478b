"""Benchmark: gated triangle attention forward + backward on one MI355X.

One step = tri_attn_fwd + tri_attn_bwd (starting node) at N=768, H=4, c=32,
bf16 inputs/outputs with fp32 accumulation, on seeded synthetic inputs that are
resident in HBM before timing starts.  Throughput uses the attention FLOP count
14*N^3*H*c (forward 4, backward 10 per logit and channel: QK^T and PV forward;
recomputed QK^T, dP, dV, dK, dQ backward).

Prints ONE JSON line.  Durations are measured with HIP events recorded on the
stream the kernels run on.  Each recorded event leaves a few microseconds of
idle time between the kernels it separates, so the timed steps carry only the
events the roofline needs (around one launch of the main backward kernel per
step); the per-stage split comes from a second pass.  The smaller
configurations (N=64 fp32, N=256, N=384 with key padding, N=640 with a wide
bias at both nodes: the crops the pages train at) are timed the same way and
reported under "configs"; ``--config i`` times only configuration i.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tri-attn fwd+bwd TFLOP/s at N=768,H=4,c=32 bf16 (% of MFMA peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class Hip:
    """Minimal HIP event API through ctypes (events on the stream torch uses).

    The events only time work on the GPU, so they are created without the
    system-scope fence: recording one then costs no cache write-back and
    invalidation between the kernels it separates.
    """

    def __init__(self, event_flags: int = HIP_EVENT_DISABLE_SYSTEM_FENCE):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.flags = event_flags
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.flags) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.lib.hipEventSynchronize(b) == 0
        assert self.lib.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "triangle_attention_tri_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, if it matches these sources."""
    try:
        with open(COUNTERS_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(x, rows: int):
    """The fp64 oracle on `rows` rows (all heads, all queries and keys) of the same workload."""
    import oracle
    n, h, _, c = x["q"].shape
    sel = slice(0, rows)
    args = (x["q"][sel], x["k"][sel], x["v"][sel], x["bias"], x["gate"][sel], None, x["dout"][sel])
    t0 = time.perf_counter()
    r = oracle.attn_bwd(*args)
    dt = time.perf_counter() - t0
    flops = 14.0 * rows * n * n * h * c
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(r["threads"]), "kind": "oracle",
            "sample": f"{rows} of {n} rows i (all {h} heads, all queries and keys), forward+backward, fp64, "
                      f"{dt:.1f} s wall"}


def time_block(lib, hip, dev, stream, n, steps, warmup, no_end):
    """The N x N x 128 block: LayerNorm + projections -> attention -> output linear, fwd + bwd.

    Every buffer is allocated before timing; a step is the six C ABI calls in
    order.  The step time comes from K bare steps; the per-call split from a
    second pass of K steps with HIP events between the calls.
    """
    import torch

    import triangle_attention_tri_amd as ta
    from triangle_attention_tri_amd import inputs
    H, c, cz = 4, 32, 128
    x = {k: v.to(dev) for k, v in inputs.block_inputs(n, cz=cz, h=H, c=c, seed=4).items()}
    e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
    q, k, v = e(n, H, n, c), e(n, H, n, c), e(n, H, n, c)
    gate, bias = e(n, n, H, c), e(H, n, n)
    mean, rstd = e(n, n, dt=torch.float32), e(n, n, dt=torch.float32)
    out, attn, lse = e(n, n, H, c), e(n, H, n, c), e(n, H, n, dt=torch.float32)
    y, d_out, dw_o = e(n, n, cz), e(n, n, H, c), e(cz, H * c)
    dq, dk, dv, dgate, dbias = e(n, H, n, c), e(n, H, n, c), e(n, H, n, c), e(n, n, H, c), e(H, n, n)
    dz, dgamma, dbeta, dw_qkvg, dw_bias = e(n, n, cz), e(cz), e(cz), e(4 * H * c, cz), e(H, cz)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sz = ctypes.c_size_t
    npair = n * n
    ws_front = torch.empty(lib.tri_attn_ln_proj_bwd_workspace_size(n, n, cz, H, c, ta.BF16), dtype=torch.uint8,
                           device=dev)
    ws_out = torch.empty(lib.tri_attn_out_proj_bwd_workspace_size(npair, H * c, cz, ta.BF16), dtype=torch.uint8,
                         device=dev)
    ws_att = torch.empty(lib.tri_attn_bwd_workspace_size(n, n, H, c, ta.BF16), dtype=torch.uint8, device=dev)
    ws_fa = torch.empty(lib.tri_attn_fwd_workspace_size(n, n, H, c, ta.BF16), dtype=torch.uint8, device=dev)
    names = ["front_fwd", "attn_fwd", "out_fwd", "out_bwd", "attn_bwd", "front_bwd"]

    def step(ending, ev):
        calls = [
            lambda: lib.tri_attn_ln_proj_fwd(n, n, cz, H, c, ta.BF16, P(x["z"]), P(x["gamma"]), P(x["beta"]),
                                             ctypes.c_float(1e-5), P(x["w_qkvg"]), P(x["w_bias"]), P(q), P(k), P(v),
                                             P(gate), P(bias), P(mean), P(rstd), stream),
            lambda: lib.tri_attn_fwd(n, n, H, c, ta.BF16, ending, P(q), P(k), P(v), P(bias), P(gate), None, P(out),
                                     P(attn), P(lse), P(ws_fa), sz(ws_fa.numel()), stream),
            lambda: lib.tri_attn_out_proj_fwd(npair, H * c, cz, ta.BF16, P(out), P(x["w_o"]), P(y), stream),
            lambda: lib.tri_attn_out_proj_bwd(npair, H * c, cz, ta.BF16, P(out), P(x["w_o"]), P(x["dy"]), P(d_out),
                                              P(dw_o), P(ws_out), sz(ws_out.numel()), stream),
            lambda: lib.tri_attn_bwd(n, n, H, c, ta.BF16, ending, P(q), P(k), P(v), P(bias), P(gate), None, P(attn),
                                     P(lse), P(d_out), P(dq), P(dk), P(dv), P(dbias), P(dgate), P(ws_att),
                                     sz(ws_att.numel()), stream),
            lambda: lib.tri_attn_ln_proj_bwd(n, n, cz, H, c, ta.BF16, P(x["z"]), P(x["gamma"]), P(x["beta"]), P(mean),
                                             P(rstd), P(x["w_qkvg"]), P(x["w_bias"]), P(dq), P(dk), P(dv), P(dgate),
                                             P(dbias), P(dz), P(dgamma), P(dbeta), P(dw_qkvg), P(dw_bias),
                                             P(ws_front), sz(ws_front.numel()), stream),
        ]
        for i, call in enumerate(calls):
            if ev is not None:
                hip.record(ev[i], stream)
            st = call()
            assert st == 0, (names[i], st)
        if ev is not None:
            hip.record(ev[len(calls)], stream)

    def run(ending, stage_times=True):
        # bare timed steps for the total; a second pass with events between the calls for the split
        for _ in range(warmup):
            step(ending, None)
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, stream)
        for _ in range(steps):
            step(ending, None)
        hip.record(t1, stream)
        torch.cuda.synchronize()
        total = hip.ms(t0, t1) / steps
        if not stage_times:
            return total, None
        evs = [[hip.event() for _ in range(len(names) + 1)] for _ in range(steps)]
        for s_ in range(steps):
            step(ending, evs[s_])
        torch.cuda.synchronize()
        stages = {nm: sum(hip.ms(ev[i], ev[i + 1]) for ev in evs) / steps for i, nm in enumerate(names)}
        return total, stages

    ms_start, stages = run(0)
    ms_end = None if no_end else run(1, stage_times=False)[0]
    attn_flops = 14.0 * n ** 3 * H * c
    lin_flops = 3 * 2.0 * npair * cz * (4 * H * c + H) + 3 * 2.0 * npair * (H * c) * cz
    # algorithmic HBM bytes of the block's streaming kernels (each tensor moved once)
    front_fwd_bytes = npair * (cz * 2 + 4 * H * c * 2 + H * 2 + 8)
    front_bwd_bytes = npair * (4 * H * c * 2 + H * 2 + cz * 2 + 8 + cz * 2)
    out_fwd_bytes = npair * (H * c * 2 + cz * 2)
    out_bwd_bytes = npair * (cz * 2 + H * c * 2 + H * c * 2)
    gbs = lambda b, ms: round(b / (ms * 1e-3) / 1e9, 1)  # noqa: E731
    return {
        "workload": f"block_N{n}_cz{cz}_H{H}_c{c}_bf16", "flops_per_step": attn_flops + lin_flops,
        "ms_per_step": round(ms_start, 4), "end_node_ms_per_step": None if ms_end is None else round(ms_end, 4),
        "tflops": round((attn_flops + lin_flops) / (ms_start * 1e-3) / 1e12, 2),
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "hbm_gbs": {"front_fwd": gbs(front_fwd_bytes, stages["front_fwd"]),
                    "front_bwd": gbs(front_bwd_bytes, stages["front_bwd"]),
                    "out_fwd": gbs(out_fwd_bytes, stages["out_fwd"]),
                    "out_bwd": gbs(out_bwd_bytes, stages["out_bwd"])},
    }


def time_chunked(lib, hip, dev, stream, n, steps, warmup, rows_list=(768, 128, 32)):
    """Chunked inference of the starting-node block at several chunk sizes: tri_attn_block_fwd_chunked
    (front end, attention, output linear) and tri_attn_block_fwd_fused (q and the gate projected inside the
    attention kernel, no saved attention), forward time per call and the workspace each needs."""
    import torch

    import triangle_attention_tri_amd as ta
    from triangle_attention_tri_amd import inputs
    H, c, cz = 4, 32, 128
    x = {k: v.to(dev) for k, v in inputs.block_inputs(n, cz=cz, h=H, c=c, seed=4).items()}
    y = torch.empty_like(x["z"])
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    res = []
    for rows in rows_list:
        rows = min(rows, n)
        entry = {"rows_per_chunk": rows}
        for kind, size_fn, fn in (("chunked", lib.tri_attn_block_fwd_chunked_workspace_size,
                                   lib.tri_attn_block_fwd_chunked),
                                  ("fused", lib.tri_attn_block_fwd_fused_workspace_size, lib.tri_attn_block_fwd_fused)):
            need = size_fn(n, cz, H, c, ta.BF16, rows)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)

            def call():
                st = fn(n, cz, H, c, ta.BF16, rows, P(x["z"]), P(x["gamma"]), P(x["beta"]), ctypes.c_float(1e-5),
                        P(x["w_qkvg"]), P(x["w_bias"]), P(x["w_o"]), None, P(y), P(ws), ctypes.c_size_t(need), stream)
                assert st == 0, (kind, st)
            for _ in range(warmup):
                call()
            t0, t1 = hip.event(), hip.event()
            torch.cuda.synchronize()
            hip.record(t0, stream)
            for _ in range(steps):
                call()
            hip.record(t1, stream)
            torch.cuda.synchronize()
            pre = "" if kind == "chunked" else "fused_"
            entry[pre + "ms"] = round(hip.ms(t0, t1) / steps, 4)
            entry[pre + "workspace_mib"] = round(need / 2 ** 20, 1)
            del ws
        res.append(entry)
    return res


def time_trimul(lib, hip, dev, stream, n, steps, warmup):
    """Triangular multiplicative update at n x n x 128 (bf16, c = 128), forward + backward, both edge directions.

    A step is tri_mul_fwd + tri_mul_bwd with every buffer allocated before timing.  K bare steps give the step
    time; K more through the profiled entry points give the split into the input side, the contraction over the
    third token (forward: T_c = A_c B_c^T; backward: dA_c = dT_c B_c and dB_c = dT_c^T A_c) and the output side.
    Each contraction is one GEMM launch of 2 n^3 c flops; its roofline is that count over its event-timed launch.
    """
    import torch

    import triangle_attention_tri_amd as ta
    from triangle_attention_tri_amd import inputs
    cz = c = 128
    x = {k: v.to(dev) for k, v in inputs.trimul_inputs(n, seed=n).items()}
    names = ta.TRIMUL_PARAMS
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sz = ctypes.c_size_t
    saved_bytes = lib.tri_mul_saved_size(n, cz, c, ta.BF16)
    ws_bytes = lib.tri_mul_workspace_size(n, cz, c, ta.BF16)
    saved = torch.empty(saved_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    y, dz = torch.empty_like(x["z"]), torch.empty_like(x["z"])
    grads = [torch.empty_like(x[k]) for k in names]
    f = ctypes.c_float(1e-5)
    vp = ctypes.c_void_p
    lib.tri_mul_fwd_profiled.argtypes = list(lib.tri_mul_fwd.argtypes) + [vp]
    lib.tri_mul_fwd_profiled.restype = ctypes.c_int
    lib.tri_mul_bwd_profiled.argtypes = list(lib.tri_mul_bwd.argtypes) + [vp]
    lib.tri_mul_bwd_profiled.restype = ctypes.c_int
    fev, bev = (ctypes.c_void_p * 4)(), (ctypes.c_void_p * 5)()

    def step(inc, fe=None, be=None):
        fa = (n, cz, c, ta.BF16, inc, P(x["z"]), *[P(x[k]) for k in names], f, P(y), P(saved), sz(saved_bytes),
              stream)
        ba = (n, cz, c, ta.BF16, inc, P(x["z"]), *[P(x[k]) for k in names], f, P(saved), sz(saved_bytes),
              P(x["dy"]), P(dz), *[P(t) for t in grads], P(ws), sz(ws_bytes), stream)
        if fe is None:
            assert lib.tri_mul_fwd(*fa) == 0
            assert lib.tri_mul_bwd(*ba) == 0
            return
        for i in range(4):
            fev[i] = fe[i]
        for i in range(5):
            bev[i] = be[i]
        assert lib.tri_mul_fwd_profiled(*fa, ctypes.cast(fev, vp)) == 0
        assert lib.tri_mul_bwd_profiled(*ba, ctypes.cast(bev, vp)) == 0

    contraction = 2.0 * n ** 3 * c
    pairs = n * n
    linear = 2.0 * pairs * cz * (4 * c + cz) * 3 + 2.0 * pairs * c * cz * 3
    out = {"workload": f"trimul_N{n}_cz{cz}_c{c}_bf16", "flops_per_step": 3 * contraction + linear,
           "contraction_flops_per_step": 3 * contraction}
    for inc in (0, 1):
        for _ in range(warmup):
            step(inc)
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, stream)
        for _ in range(steps):
            step(inc)
        hip.record(t1, stream)
        torch.cuda.synchronize()
        ms = hip.ms(t0, t1) / steps
        st = dict(front_fwd=0.0, contract_fwd=0.0, back_fwd=0.0, back_bwd=0.0, contract_da=0.0, contract_db=0.0,
                  front_bwd=0.0)
        for _ in range(steps):
            fe = [hip.event() for _ in range(4)]
            be = [hip.event() for _ in range(5)]
            step(inc, fe, be)
            torch.cuda.synchronize()
            for key, (a, b) in zip(("front_fwd", "contract_fwd", "back_fwd"), ((fe[0], fe[1]), (fe[1], fe[2]),
                                                                              (fe[2], fe[3]))):
                st[key] += hip.ms(a, b) / steps
            for key, (a, b) in zip(("back_bwd", "contract_da", "contract_db", "front_bwd"),
                                   ((be[0], be[1]), (be[1], be[2]), (be[2], be[3]), (be[3], be[4]))):
                st[key] += hip.ms(a, b) / steps
        launch = {k: st[k] for k in ("contract_fwd", "contract_da", "contract_db")}
        kmax = max(launch, key=launch.get)
        ach = contraction / (launch[kmax] * 1e-3) / 1e12
        out["incoming" if inc else "outgoing"] = {
            "ms_per_step": round(ms, 4), "tflops": round(out["flops_per_step"] / (ms * 1e-3) / 1e12, 2),
            "stages_ms": {k: round(v, 4) for k, v in st.items()},
            "contraction_roofline": {"kernel": "gemm_kernel (per-channel contraction, " + kmax + ")",
                                     "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                                     "launch_ms": round(launch[kmax], 4)}}
    return out


class AttnCase:
    """One attention workload resident on the GPU: seeded inputs, outputs, workspaces and the C ABI calls of a
    step (tri_attn_fwd + tri_attn_bwd, or the residual-compensated pair)."""

    def __init__(self, lib, hip, dev, stream, n, dtype, seed, bias_std=1.0, valid_len=None, H=4, c=32):
        import torch

        import triangle_attention_tri_amd as ta
        from triangle_attention_tri_amd import inputs
        self.lib, self.hip, self.stream, self.n, self.H, self.c = lib, hip, stream, n, H, c
        self.dt = ta.BF16 if dtype == torch.bfloat16 else ta.F32
        self.xc = inputs.attn_inputs(n, H, c, dtype, seed=seed, bias_std=bias_std, valid_len=valid_len)
        x = self.x = {k: (None if v is None else v.to(dev)) for k, v in self.xc.items()}
        self.valid = n if valid_len is None else valid_len
        self.out = torch.empty_like(x["gate"])
        self.attn = torch.empty_like(x["q"])
        self.lse = torch.empty((n, H, n), dtype=torch.float32, device=dev)
        self.grads = [torch.empty_like(x[k]) for k in ("q", "k", "v", "bias", "gate")]
        self.ws_bytes = ta.workspace_size(n, n, H, c, dtype)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.fws_bytes = ta.fwd_workspace_size(n, n, H, c, dtype)
        self.fws = torch.empty(self.fws_bytes, dtype=torch.uint8, device=dev)
        self.chunk = ta.bwd_chunk_rows(n, n, H, c, dtype)
        self.chunks = -(-n // self.chunk)
        self.res = torch.empty((n, H, n, c), dtype=torch.int8, device=dev) if self.dt == ta.BF16 else None
        self.events = (ctypes.c_void_p * (4 * self.chunks))()
        lib.tri_attn_bwd_profiled.argtypes = list(lib.tri_attn_bwd.argtypes) + [ctypes.c_void_p]
        lib.tri_attn_bwd_profiled.restype = ctypes.c_int

    def step(self, ending: int, fwd_ev=None, bwd_ev=None, rc: bool = False):
        """fwd_ev: (before, after) the forward or None; bwd_ev: 4 events per backward chunk (None entries skipped)
        or None for the plain entry point."""
        P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
        x, n, H, c, lib, st = self.x, self.n, self.H, self.c, self.lib, self.stream
        sz = ctypes.c_size_t
        if fwd_ev is not None and fwd_ev[0] is not None:
            self.hip.record(fwd_ev[0], st)
        if rc:
            r = lib.tri_attn_fwd_rc(n, n, H, c, self.dt, ending, P(x["q"]), P(x["k"]), P(x["v"]), P(x["bias"]),
                                    P(x["gate"]), P(x["mask"]), P(self.out), P(self.attn), P(self.res), P(self.lse),
                                    P(self.fws), sz(self.fws_bytes), st)
        else:
            r = lib.tri_attn_fwd(n, n, H, c, self.dt, ending, P(x["q"]), P(x["k"]), P(x["v"]), P(x["bias"]),
                                 P(x["gate"]), P(x["mask"]), P(self.out), P(self.attn), P(self.lse), P(self.fws),
                                 sz(self.fws_bytes), st)
        assert r == 0, r
        if fwd_ev is not None and fwd_ev[1] is not None:
            self.hip.record(fwd_ev[1], st)
        g = [P(t) for t in self.grads]
        if rc:
            r = lib.tri_attn_bwd_rc(n, n, H, c, self.dt, ending, P(x["q"]), P(x["k"]), P(x["v"]), P(x["bias"]),
                                    P(x["gate"]), P(x["mask"]), P(self.attn), P(self.res), P(self.lse),
                                    P(x["dout"]), *g, P(self.ws), sz(self.ws_bytes), st)
            assert r == 0, r
            return
        common = (n, n, H, c, self.dt, ending, P(x["q"]), P(x["k"]), P(x["v"]), P(x["bias"]), P(x["gate"]),
                  P(x["mask"]), P(self.attn), P(self.lse), P(x["dout"]), *g, P(self.ws), sz(self.ws_bytes), st)
        if bwd_ev is None:
            r = lib.tri_attn_bwd(*common)
        else:
            for i in range(4 * self.chunks):
                self.events[i] = bwd_ev[i]
            r = lib.tri_attn_bwd_profiled(*common, ctypes.cast(self.events, ctypes.c_void_p))
        assert r == 0, r

    def timed(self, ending: int, steps: int, warmup: int, stages: bool = True):
        """K timed steps carrying only two events each, around one launch of the main backward kernel (its
        launch time, for the roofline; the chunks take turns), then (stages=True) K steps with events between
        every stage.  Each recorded event leaves a few microseconds of idle time between the kernels it
        separates, which is why the timed steps carry no others."""
        import torch
        hip, ch = self.hip, self.chunks
        for _ in range(warmup):
            self.step(ending)
        torch.cuda.synchronize()
        # one chunk's launch per step carries the two events (chunks in rotation), so every step has the same
        # two idle gaps whatever the chunk count
        main_ev = [(hip.event(), hip.event()) for _ in range(steps)]
        bwd_ev = []
        for s_ in range(steps):
            evs = [None] * (4 * ch)
            m = s_ % ch
            evs[4 * m + 1], evs[4 * m + 2] = main_ev[s_]
            bwd_ev.append(evs)
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, self.stream)
        for s_ in range(steps):
            self.step(ending, bwd_ev=bwd_ev[s_])
        hip.record(t1, self.stream)
        torch.cuda.synchronize()
        total = hip.ms(t0, t1) / steps
        launches = [hip.ms(a, b) for (a, b) in main_ev]
        out = {"ms": total, "main_launch_ms": sum(launches) / len(launches), "main_launches_per_step": ch}
        if stages:
            st = {"fwd": 0.0, "bwd_pre": 0.0, "bwd_main": 0.0, "bwd_reduce": 0.0}
            for _ in range(steps):
                fe = (hip.event(), hip.event())
                be = [hip.event() for _ in range(4 * ch)]
                self.step(ending, fwd_ev=fe, bwd_ev=be)
                torch.cuda.synchronize()
                st["fwd"] += hip.ms(fe[0], fe[1])
                for m in range(ch):
                    st["bwd_pre"] += hip.ms(be[4 * m], be[4 * m + 1])
                    st["bwd_main"] += hip.ms(be[4 * m + 1], be[4 * m + 2])
                    st["bwd_reduce"] += hip.ms(be[4 * m + 2], be[4 * m + 3])
            out["stages"] = {k: v / steps for k, v in st.items()}
        return out

    def flops(self):
        """fwd + bwd: 4 + 10 flops per logit and channel over the valid keys (one recompute of P)."""
        return 14.0 * self.n * self.n * self.valid * self.H * self.c

    def main_flops_per_launch(self):
        return 10.0 * self.chunk * self.n * self.valid * self.H * self.c


def main_kernel_name(case):
    return "bwd_group_kernel" if case.dt == 1 else ("bwd_tile_kernel" if case.n <= 256 else "bwd_main_kernel")


def config_line(case, res, workload, peak, node):
    """Per-configuration record: the step, the forward and backward stages and the main backward kernel against
    its roofline (its own algorithmic flops per launch over its event-timed launch duration)."""
    ms = res["ms"]
    tf = case.flops() / (ms * 1e-3) / 1e12
    ach = case.main_flops_per_launch() / (res["main_launch_ms"] * 1e-3) / 1e12
    return {"workload": workload, "n": case.n, "node": node, "dtype": "bf16" if case.dt == 1 else "f32",
            "valid_keys": case.valid, "flops_per_step": case.flops(), "ms_per_step": round(ms, 4),
            "tflops": round(tf, 2), "peak_tflops": peak, "frac_of_peak": round(tf / peak, 4),
            "stages_ms": {k: round(v, 4) for k, v in res.get("stages", {}).items()},
            "main_kernel": {"kernel": main_kernel_name(case), "launch_ms": round(res["main_launch_ms"], 4),
                            "launches_per_step": res["main_launches_per_step"], "rows_per_launch": case.chunk,
                            "achieved_tflops": round(ach, 2), "frac": round(ach / peak, 4)}}


# The configurations of this workload (seeded as in the tests); index 4 is the headline.
CONFIGS = {
    0: dict(n=64, dtype="f32", seed=0, workload="tri_attn_start_fwd_bwd_N64_H4_c32_f32", nodes=(0,)),
    1: dict(n=256, dtype="bf16", seed=1, workload="tri_attn_start_fwd_bwd_N256_H4_c32_bf16", nodes=(0,)),
    2: dict(n=384, dtype="bf16", seed=2, valid_len=345,
            workload="tri_attn_start_fwd_bwd_N384_H4_c32_bf16_keymask345", nodes=(0,)),
    3: dict(n=640, dtype="bf16", seed=3, bias_std=2.0, workload="tri_attn_fwd_bwd_N640_H4_c32_bf16_bias_std2",
            nodes=(0, 1)),
}
PEAK_FP32_TFLOPS = 157.3


def time_configs(lib, hip, dev, stream, which, steps, warmup):
    import torch
    lines = []
    for idx in which:
        cfg = CONFIGS[idx]
        dtype = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
        case = AttnCase(lib, hip, dev, stream, cfg["n"], dtype, cfg["seed"], cfg.get("bias_std", 1.0),
                        cfg.get("valid_len"))
        peak = PEAK_BF16_TFLOPS if cfg["dtype"] == "bf16" else PEAK_FP32_TFLOPS
        for node in cfg["nodes"]:
            res = case.timed(node, steps, warmup)
            line = config_line(case, res, cfg["workload"], peak, "end" if node else "start")
            line["config"] = idx
            lines.append(line)
        del case
        torch.cuda.empty_cache()
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--n", type=int, default=768)
    ap.add_argument("--config", type=int, default=None, choices=sorted(CONFIGS),
                    help="time only this smaller configuration and print its record (for profiling runs)")
    ap.add_argument("--cpu-rows", type=int, default=512, help="rows of the oracle CPU sample (0 = skip)")
    ap.add_argument("--no-end", action="store_true", help="skip the ending-node timing")
    ap.add_argument("--no-rc", action="store_true", help="skip the timing of the residual-compensated pair")
    ap.add_argument("--no-chunked", action="store_true", help="skip the chunked block inference timing")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the LayerNorm + projection + attention + output-linear block timing")
    ap.add_argument("--no-configs", action="store_true", help="skip the smaller configurations")
    ap.add_argument("--no-trimul", action="store_true", help="skip the triangular multiplicative update timing")
    ap.add_argument("--trimul-only", action="store_true", help="time only the triangular multiplicative update")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported on this single-GPU build",
              file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import torch

    import triangle_attention_tri_amd as ta

    lib = ta.load()
    hip = Hip()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    if args.copy_calibration_mib > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters scale the HBM byte counts
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.trimul_only:
        print(json.dumps(time_trimul(lib, hip, dev, stream, args.n, args.steps, args.warmup)), flush=True)
        return

    if args.config is not None:
        for line in time_configs(lib, hip, dev, stream, [args.config], args.steps, args.warmup):
            print(json.dumps(line), flush=True)
        return

    n, H, c = args.n, 4, 32
    case = AttnCase(lib, hip, dev, stream, n, torch.bfloat16, seed=4)
    res = case.timed(0, args.steps, args.warmup)
    ms_step = res["ms"]
    flops = case.flops()
    value = flops / (ms_step * 1e-3) / 1e12

    # roofline of the kernel that takes the most time, the main backward kernel (twice the forward's time at
    # this size): the algorithmic flops of one launch (10 per logit and channel over the launch's row chunk)
    # over its average launch duration, from the events around each launch in the timed steps
    work = case.main_flops_per_launch()
    achieved = work / (res["main_launch_ms"] * 1e-3) / 1e12
    kernel = "bwd_group_kernel"
    roofline = {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(kernel), "launch_ms": round(res["main_launch_ms"], 4),
                "launches_per_step": res["main_launches_per_step"], "rows_per_launch": case.chunk}

    end_ms = None
    if not args.no_end:
        end_ms = case.timed(1, max(3, args.steps // 2), 2, stages=False)["ms"]

    rc_ms = None
    if not args.no_rc:
        rc_steps = max(3, args.steps // 2)
        for _ in range(2):
            case.step(0, rc=True)
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, stream)
        for _ in range(rc_steps):
            case.step(0, rc=True)
        hip.record(t1, stream)
        torch.cuda.synchronize()
        rc_ms = hip.ms(t0, t1) / rc_steps
    xc = case.xc
    del case
    torch.cuda.empty_cache()

    block = None if args.no_block else time_block(lib, hip, dev, stream, n, max(3, args.steps // 2), 2, args.no_end)
    chunked = None if args.no_chunked else time_chunked(lib, hip, dev, stream, n, 5, 2)
    configs = None if args.no_configs else time_configs(lib, hip, dev, stream, sorted(CONFIGS),
                                                        max(5, args.steps // 2), 3)
    trimul = None if args.no_trimul else time_trimul(lib, hip, dev, stream, n, max(3, args.steps // 4), 2)

    cpu = None
    if rank == 0 and args.cpu_rows > 0:
        cpu = cpu_baseline(xc, min(args.cpu_rows, n))

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"tri_attn_start_fwd_bwd_N{n}_H{H}_c{c}_bf16", "n": n, "h": H, "c": c,
                   "node": "start", "mask": None, "flops_per_step": flops},
        "pct_of_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "stages_ms": {k: round(v, 4) for k, v in res["stages"].items()},
        "end_node_ms_per_step": None if end_ms is None else round(end_ms, 4),
        "residual_compensated_ms_per_step": None if rc_ms is None else round(rc_ms, 4),
        "roofline": roofline,
        "configs": configs,
        "trimul": trimul,
        "block": block,
        "chunked_block_fwd": chunked,
        "cpu_baseline": cpu,
    }
    if rank == 0:
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
