"""Benchmark: gated triangle attention forward + backward on one MI355X.

One step = tri_attn_fwd + tri_attn_bwd (starting node) at N=768, H=4, c=32,
bf16 inputs/outputs with fp32 accumulation, on seeded synthetic inputs that are
resident in HBM before timing starts.  Throughput uses the attention FLOP count
14*N^3*H*c (forward 4, backward 10 per logit and channel: QK^T and PV forward;
recomputed QK^T, dP, dV, dK, dQ backward).

Prints ONE JSON line.  Durations are measured with HIP events recorded on the
stream the kernels run on.  Each recorded event leaves a few microseconds of
idle time between the kernels it separates, so the timed steps carry only the
events the roofline needs (around the main backward kernel); the per-stage
split comes from a second pass.
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
    """Chunked inference of the starting-node block (tri_attn_block_fwd_chunked) at several chunk sizes:
    forward time per call and the workspace it needs, next to the unchunked forward's intermediates."""
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
        need = lib.tri_attn_block_fwd_chunked_workspace_size(n, cz, H, c, ta.BF16, rows)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

        def call():
            st = lib.tri_attn_block_fwd_chunked(n, cz, H, c, ta.BF16, rows, P(x["z"]), P(x["gamma"]), P(x["beta"]),
                                                ctypes.c_float(1e-5), P(x["w_qkvg"]), P(x["w_bias"]), P(x["w_o"]),
                                                None, P(y), P(ws), ctypes.c_size_t(need), stream)
            assert st == 0, st
        for _ in range(warmup):
            call()
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, stream)
        for _ in range(steps):
            call()
        hip.record(t1, stream)
        torch.cuda.synchronize()
        res.append({"rows_per_chunk": rows, "ms": round(hip.ms(t0, t1) / steps, 4),
                    "workspace_mib": round(need / 2 ** 20, 1)})
        del ws
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--n", type=int, default=768)
    ap.add_argument("--cpu-rows", type=int, default=512, help="rows of the oracle CPU sample (0 = skip)")
    ap.add_argument("--no-end", action="store_true", help="skip the ending-node timing")
    ap.add_argument("--no-rc", action="store_true", help="skip the timing of the residual-compensated pair")
    ap.add_argument("--no-chunked", action="store_true", help="skip the chunked block inference timing")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the LayerNorm + projection + attention + output-linear block timing")
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
    from triangle_attention_tri_amd import inputs

    lib = ta.load()
    hip = Hip()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n, H, c = args.n, 4, 32
    xc = inputs.attn_inputs(n, H, c, torch.bfloat16, seed=4)
    xd = {k: (None if v is None else v.to(dev)) for k, v in xc.items()}
    out = torch.empty_like(xd["gate"])
    attn = torch.empty((n, H, n, c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((n, H, n), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(xd[k]) for k in ("q", "k", "v"))
    dbias, dgate = torch.empty_like(xd["bias"]), torch.empty_like(xd["gate"])
    ws_bytes = ta.workspace_size(n, n, H, c, torch.bfloat16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fws_bytes = ta.fwd_workspace_size(n, n, H, c, torch.bfloat16)
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    attn_res = torch.empty((n, H, n, c), dtype=torch.int8, device=dev)
    bwd_events = (ctypes.c_void_p * 4)()
    lib.tri_attn_bwd_profiled.argtypes = list(lib.tri_attn_bwd.argtypes) + [ctypes.c_void_p]
    lib.tri_attn_bwd_profiled.restype = ctypes.c_int

    def step(ending: int, ev=None, rc: bool = False):
        if ev is not None and ev[0] is not None:
            hip.record(ev[0], stream)
        if rc:  # residual-compensated pair (tri_attn_fwd_rc / tri_attn_bwd_rc)
            st = lib.tri_attn_fwd_rc(n, n, H, c, ta.BF16, ending, P(xd["q"]), P(xd["k"]), P(xd["v"]), P(xd["bias"]),
                                     P(xd["gate"]), None, P(out), P(attn), P(attn_res), P(lse), P(fws),
                                     ctypes.c_size_t(fws_bytes), stream)
            assert st == 0, st
            st = lib.tri_attn_bwd_rc(n, n, H, c, ta.BF16, ending, P(xd["q"]), P(xd["k"]), P(xd["v"]), P(xd["bias"]),
                                     P(xd["gate"]), None, P(attn), P(attn_res), P(lse), P(xd["dout"]), P(dq), P(dk),
                                     P(dv), P(dbias), P(dgate), P(ws), ctypes.c_size_t(ws_bytes), stream)
            assert st == 0, st
            return
        st = lib.tri_attn_fwd(n, n, H, c, ta.BF16, ending, P(xd["q"]), P(xd["k"]), P(xd["v"]), P(xd["bias"]),
                              P(xd["gate"]), None, P(out), P(attn), P(lse), P(fws), ctypes.c_size_t(fws_bytes), stream)
        assert st == 0, st
        common = (n, n, H, c, ta.BF16, ending, P(xd["q"]), P(xd["k"]), P(xd["v"]), P(xd["bias"]), P(xd["gate"]),
                  None, P(attn), P(lse), P(xd["dout"]), P(dq), P(dk), P(dv), P(dbias), P(dgate), P(ws),
                  ctypes.c_size_t(ws_bytes), stream)
        if ev is None:
            st = lib.tri_attn_bwd(*common)
        else:
            for i in range(4):
                bwd_events[i] = ev[1 + i]  # None: not recorded
            st = lib.tri_attn_bwd_profiled(*common, ctypes.cast(bwd_events, ctypes.c_void_p))
        assert st == 0, st

    def timed(ending: int, steps: int, warmup: int):
        """K timed steps, then K more with events between every stage.

        Each recorded event leaves a few microseconds of idle time between the
        kernels it separates, so the timed steps record only the two events
        around the main backward kernel (its launch time, for the roofline).
        The per-stage split comes from the second, separately timed pass.
        """
        for _ in range(warmup):
            step(ending)
        torch.cuda.synchronize()
        main_ev = [(hip.event(), hip.event()) for _ in range(steps)]
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, stream)
        for s in range(steps):
            step(ending, (None, None, main_ev[s][0], main_ev[s][1], None))
        hip.record(t1, stream)
        torch.cuda.synchronize()
        total = hip.ms(t0, t1)
        main_ms = sum(hip.ms(a, b) for a, b in main_ev) / steps
        evs = [[hip.event() for _ in range(5)] for _ in range(steps)]
        for s in range(steps):
            step(ending, evs[s])
        torch.cuda.synchronize()
        stages = {"fwd": 0.0, "bwd_pre": 0.0, "bwd_main": 0.0, "dbias_reduce": 0.0}
        for e in evs:
            stages["fwd"] += hip.ms(e[0], e[1])
            stages["bwd_pre"] += hip.ms(e[1], e[2])
            stages["bwd_main"] += hip.ms(e[2], e[3])
            stages["dbias_reduce"] += hip.ms(e[3], e[4])
        return total / steps, {k: v / steps for k, v in stages.items()}, main_ms

    if args.copy_calibration_mib > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters scale the HBM byte counts
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_step, stages, main_ms = timed(0, args.steps, args.warmup)
    flops = 14.0 * n ** 3 * H * c
    value = flops / (ms_step * 1e-3) / 1e12

    # roofline of the kernel that takes the most time: the main backward kernel (twice the forward's time at
    # this size), its launch time measured by the events around it in the timed steps
    work = 10.0 * n ** 3 * H * c
    achieved = work / (main_ms * 1e-3) / 1e12
    kernel = "bwd_group_kernel"
    roofline = {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(kernel), "launch_ms": round(main_ms, 4)}

    end_ms = None
    if not args.no_end:
        end_ms = timed(1, max(3, args.steps // 2), 2)[0]

    rc_ms = None
    if not args.no_rc:
        rc_steps = max(3, args.steps // 2)
        for _ in range(2):
            step(0, rc=True)
        t0, t1 = hip.event(), hip.event()
        torch.cuda.synchronize()
        hip.record(t0, stream)
        for _ in range(rc_steps):
            step(0, rc=True)
        hip.record(t1, stream)
        torch.cuda.synchronize()
        rc_ms = hip.ms(t0, t1) / rc_steps

    block = None if args.no_block else time_block(lib, hip, dev, stream, n, max(3, args.steps // 2), 2, args.no_end)
    chunked = None if args.no_chunked else time_chunked(lib, hip, dev, stream, n, 3, 1)

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
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "end_node_ms_per_step": None if end_ms is None else round(end_ms, 4),
        "residual_compensated_ms_per_step": None if rc_ms is None else round(rc_ms, 4),
        "roofline": roofline,
        "block": block,
        "chunked_block_fwd": chunked,
        "cpu_baseline": cpu,
    }
    if rank == 0:
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
