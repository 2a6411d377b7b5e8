#!/usr/bin/env python3
"""MXFP4 MoE layer benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one moe_mxfp4_forward call (router + top-k/softmax, expert
grouping, gate_up grouped GEMM with fused SwiGLU, down grouped GEMM,
combine; plus the FP8 quantisation of x in FP8 mode) over one batch whose
inputs already sit in HBM.  W untimed steps, then K timed steps between
two device synchronisations; value = tokens / second of the timed steps.
Weights are cycled over enough identical copies that a step does not find
its experts in the 256 MB Infinity Cache left by the previous ones.

The per-stage durations come from HIP events the library records on its
stream inside the timed steps; the dominant kernel's average duration
gives the roofline fraction against MI355X's published peaks.  The CPU
baseline is the float64 oracle timed on a bounded slice of the same
workload on the host cores (a reported baseline, not the target).

Workloads (synthetic, seeded; see workloads/):
  prefill_120b_t4096   gpt-oss-120b MoE layer, E=128, top-4, H=I=2880, T=4096, bf16 (default)
  decode_20b_t{1,8,64} gpt-oss-20b MoE layer, E=32, top-4, H=I=2880, bf16
  fp8_20b_t2048        W-MXFP4 A-FP8, gpt-oss-20b shape, T=2048
  tiny                 E=4, top-2, H=I=64, T=8, fp32
  unpack_20b           mxfp4_unpack of the 20b expert tensors to bf16 (GB/s)
  linear_t4096_k2880_n5760  weight-only MXFP4 dense layer y = x W^T + b, bf16
  fp8_linear_t4096_k2880_n5760  FP8 E4M3 W8A8 dense layer, static per-tensor scales
  bf16_20b_t{T}        the 20b layer at any T (with --path dense: the all-experts path)
  int8_20b_t{T}        INT8 W8A8 MoE layer (per-channel weights, per-token activations), 20b shape
                       (T=2048 prefill; T <= 128 runs the decode-shaped kernels)
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MXFP4 MoE layer tokens/s; % HBM roofline (decode), % MFMA peak (prefill)"
PEAK = {"hbm_GBps": 8000.0, "bf16_TFLOPs": 2500.0, "fp8_TFLOPs": 5000.0, "int8_TOPs": 5000.0, "fp32_TFLOPs": 157.3}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
EV_EVERY = 4  # timed steps between two recordings of the dominant stage's events
GRAPH_STEPS = 20  # forwards captured per HIP graph in the graph launch mode
# the GEMM and codec kernels and what decides their work items (the grouping
# writes the token tiles and item records the GEMMs read)
KERNEL_SOURCES = ["mxfp4_quantized_moe_amd/csrc/moe_gemm.hip", "mxfp4_quantized_moe_amd/csrc/codec.hip",
                  "mxfp4_quantized_moe_amd/csrc/device_common.h", "mxfp4_quantized_moe_amd/csrc/gemm_common.h",
                  "mxfp4_quantized_moe_amd/csrc/decode_tile.h", "mxfp4_quantized_moe_amd/csrc/routing.hip",
                  "mxfp4_quantized_moe_amd/csrc/xcd_split.h", "mxfp4_quantized_moe_amd/csrc/launch.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ HIP events

class HipEvents:
    """hipEvent_t handles from libamdhip64 (the stream-ordered timers the
    library records around its stages)."""

    _hip = None

    def __init__(self, n: int, only=None):
        if HipEvents._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvents._hip = hip
        self.hip = HipEvents._hip
        self.arr = (ctypes.c_void_p * n)()  # entries left NULL are not recorded
        for i in range(n):
            if only is not None and i not in only:
                continue
            h = ctypes.c_void_p()
            # device-scope release: a timing marker without a system-wide cache flush
            if self.hip.hipEventCreateWithFlags(ctypes.byref(h), 0x40000000) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = h
        self.n = n

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for i in range(self.n):
            if self.arr[i]:
                self.hip.hipEventDestroy(self.arr[i])


# ------------------------------------------------------------ workloads

def make_case(name: str):
    import workloads as W

    if name == "prefill_120b_t4096":
        return W.prefill_120b()
    if name.startswith("decode_20b_t"):
        return W.decode_20b(T=int(name.rsplit("t", 1)[1]))
    if name == "fp8_20b_t2048":
        return W.fp8_20b()
    if name.startswith("bf16_20b_t"):
        return W.bf16_20b(T=int(name.rsplit("t", 1)[1]))
    if name == "tiny":
        return W.tiny()
    raise SystemExit(f"unknown workload {name}")


def layer_bytes(layer) -> int:
    return sum(a.nbytes for a in (layer.gate_up_blocks, layer.gate_up_scales, layer.gate_up_bias, layer.down_blocks,
                                  layer.down_scales, layer.down_bias))


def expert_gemm_bytes(case, phase: int, n_active: int, dense: bool = False) -> int:
    """Algorithmic HBM bytes of one grouped-GEMM launch: the routed experts'
    packed weights, scales and biases once, the activations in and out once
    (rows per token: top_k routed, E dense)."""
    L = case.layer
    H, I, T = L.H, L.I, case.T
    k = L.E if dense else L.top_k
    pb = 2 if L.param_dtype == "bf16" else 4
    ab = 1 if case.fp8 else (2 if case.act_dtype == "bf16" else 4)
    if phase == 0:
        w = 2 * I * (H // 32) * 17 + 2 * I * pb
        return n_active * w + T * H * ab + T * k * I * ab
    w = H * (I // 32) * 17 + H * pb
    yb = 2 if case.act_dtype == "bf16" else 4  # Y: bf16 with bf16 activations, else fp32
    return n_active * w + T * k * I * ab + T * k * H * yb


def step_bytes(case, n_active: int) -> int:
    """Algorithmic HBM bytes of one whole routed step: the router's weights
    and bias, x in, the routed experts' packed weights, scales and biases of
    both matrices once, and the output (the intermediates h and Y need not
    leave the chip)."""
    L = case.layer
    H, I, T = L.H, L.I, case.T
    pb = 2 if L.param_dtype == "bf16" else 4
    ab = 2 if case.act_dtype == "bf16" else 4  # x and out stay bf16 in the FP8 mode
    expert = 2 * I * (H // 32) * 17 + 2 * I * pb + H * (I // 32) * 17 + H * pb
    return L.E * H * pb + L.E * pb + n_active * expert + 2 * T * H * ab


def expert_gemm_flops(case, phase: int, dense: bool = False) -> int:
    L = case.layer
    slots = case.T * (L.E if dense else L.top_k)
    return 2 * slots * (2 * L.I) * L.H if phase == 0 else 2 * slots * L.H * L.I


def cpu_baseline(case, budget_s: float, dense: bool = False):
    """The oracle as it stands on a bounded token slice of the workload (its
    all-experts forward for the dense path)."""
    import numpy as np

    import oracle as O
    import workloads as W

    try:
        from threadpoolctl import threadpool_info

        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        cores = int(info[0]["num_threads"]) if info else os.cpu_count()
        blas = info[0].get("internal_api", "blas") if info else "unknown"
    except Exception:
        cores, blas = os.cpu_count(), "unknown"
    scales = {}
    if case.fp8:
        s_x, s_h = O.calibrate_fp8(case.layer, case.x_calib, "bf16")
        scales = dict(fp8=True, x_scale=s_x, h_scale=s_h)
    n = 1
    elapsed = 0.0
    done = 0
    # grow the slice until the budget is used (each slice is an independent forward)
    while True:
        rows = np.arange(done, min(done + n, case.T))
        if rows.size == 0:
            break
        sub = W.MoECase(case.name, case.layer, case.x[rows].copy(), case.act_dtype, case.fp8, case.x_calib)
        t0 = time.perf_counter()
        if dense and not case.fp8:
            O.moe_forward_dense(sub.layer, sub.x, sub.act_dtype)
        else:
            O.moe_forward(sub.layer, sub.x, sub.act_dtype, **scales)
        elapsed += time.perf_counter() - t0
        done += rows.size
        if elapsed >= budget_s or done >= case.T:
            break
        n = min(n * 2, case.T - done)
    return {"value": done / elapsed, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {done} of {case.T} tokens of {case.name}, float64 NumPy ({blas}), "
                      f"{elapsed:.1f} s, slices of doubling size each dequantising "
                      f"{'every expert' if dense and not case.fp8 else 'their routed experts'}"}


def oracle_slices(fn, total: int, budget_s: float, what: str) -> dict:
    """The oracle as it stands, fn(lo, hi) on slices [lo, hi) of `total`
    rows of doubling size until about budget_s seconds are used.  Returns
    rows per second with the sample description."""
    try:
        from threadpoolctl import threadpool_info

        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        cores = int(info[0]["num_threads"]) if info else os.cpu_count()
        blas = info[0].get("internal_api", "blas") if info else "unknown"
    except Exception:
        cores, blas = os.cpu_count(), "unknown"
    n, done, elapsed = 1, 0, 0.0
    while done < total:
        hi = min(done + n, total)
        t0 = time.perf_counter()
        fn(done, hi)
        elapsed += time.perf_counter() - t0
        done = hi
        if elapsed >= budget_s:
            break
        n = min(n * 2, total - done)
    return {"rows_per_s": done / elapsed, "cores": cores, "kind": "oracle",
            "sample": f"first {done} of {total} {what}, float64 NumPy ({blas}), {elapsed:.1f} s, slices of doubling size"}


# ------------------------------------------------------------ main legs

def bench_layer(args, dev):
    import numpy as np
    import torch

    import mxfp4_quantized_moe_amd as mx
    import workloads as W
    from mxfp4_quantized_moe_amd.binding import STAGE_EVENTS, STAGES

    case = make_case(args.workload)
    L = case.layer
    T = case.T
    w0 = W.layer_to_torch(L, dev)
    if args.layout == "tiled":
        w0 = w0.tiled()  # the one-time load step of a serving setup, outside the timed region
        torch.cuda.synchronize()
    x = W.array_to_torch(case.x, dev)
    _, _, counts, _, _, _ = mx.moe_mxfp4_route(w0, x)
    dense = args.path == "dense"
    n_active = L.E if dense else int((W.torch_to_array(counts) > 0).sum())
    # identical weight copies: enough that a copy's routed experts were last
    # read more than 1 GB of traffic ago (past the 256 MB Infinity Cache)
    per_step = n_active * layer_bytes(L) // L.E
    copies = min(64, -(-int(1.0e9) // per_step) + 1) if args.copies is None else args.copies
    weights = [w0] + [type(w0)(*[getattr(w0, f).clone() for f in ("gate_up_blocks", "gate_up_scales", "gate_up_bias",
                                                                  "down_blocks", "down_scales", "down_bias",
                                                                  "router_w", "router_b")],
                                     top_k=w0.top_k, layout=w0.layout)
                      for _ in range(copies - 1)]
    fp8_kw = {}
    if case.fp8:
        sc = mx.moe_mxfp4_calibrate_fp8(weights[0], W.array_to_torch(case.x_calib, dev))
        s = W.torch_to_array(sc)
        fp8_kw = dict(fp8=True, x_scale=float(s[0]), h_scale=float(s[1]))
    ws = mx.alloc_workspace(weights[0], T, x.dtype, case.fp8, dense)
    out = torch.empty_like(x)
    fp8_kw["dense"] = dense

    # a plain copy of known size: the reference point that scales the HBM
    # byte counters of a profiled run (bytes moved = 2 x 256 MiB)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    del src, dst

    # one prepared call per weight copy: the tensors are checked once, so a
    # timed step costs the host only the library call itself
    plans = [mx.ForwardPlan(w, x, out=out, workspace=ws, **fp8_kw) for w in weights]
    for i in range(args.warmup):
        plans[i % copies]()
    torch.cuda.synchronize()

    # timed steps: the two events around the dominant stage (gate_up +
    # SwiGLU) are recorded on every EV_EVERY-th step only: each record costs
    # stream time (a few microseconds, a fifth of a one-token step)
    GU = STAGES.index("gate_up_swiglu")
    timed = list(range(0, args.steps, EV_EVERY))

    def run_steps(launch: str):
        """K timed forwards; returns (seconds, gate_up ms of the recorded
        steps).  graph: the forwards are captured GRAPH_STEPS at a time into
        HIP graphs before the clock starts and the timed region replays the
        graphs, so the host's per-launch cost leaves the measurement (events
        recorded inside a graph give no elapsed times, so none are);
        eager: one library call per forward, with the gate_up events."""
        ev = {i: HipEvents(STAGE_EVENTS, only=(GU, GU + 1)) for i in timed} if launch == "eager" else {}
        graphs = []
        if launch == "graph":
            cs = torch.cuda.Stream()
            for g0 in range(0, args.steps, GRAPH_STEPS):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    for i in range(g0, min(args.steps, g0 + GRAPH_STEPS)):
                        plans[i % copies](stage_events=ev[i].arr if i in ev else None)
                graphs.append(g)
            for g in graphs[:1]:  # one untimed replay (first-launch set-up of the graph)
                g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if launch == "graph":
            for g in graphs:
                g.replay()
        else:
            for i in range(args.steps):
                plans[i % copies](stage_events=ev[i].arr if i in ev else None)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gu = np.array([e.elapsed_ms(GU, GU + 1) for e in ev.values()])
        for e in ev.values():
            e.close()
        del graphs
        return t1 - t0, gu

    # the eager steps time the dominant kernel; in the graph mode the
    # graph replays then give the throughput
    te, gu_ms = run_steps("eager")
    eager = {"value": T * args.steps / te, "ms_per_step": te * 1e3 / args.steps}
    dt = run_steps("graph")[0] if args.launch == "graph" else te
    ms_step = dt * 1e3 / args.steps

    # per-stage breakdown from a separate, untimed pass with every event
    nb = min(args.steps, 10)
    evb = [HipEvents(STAGE_EVENTS) for _ in range(nb)]
    for i in range(nb):
        plans[i % copies](stage_events=evb[i].arr)
    torch.cuda.synchronize()
    avg = np.array([[e.elapsed_ms(j, j + 1) for j in range(STAGE_EVENTS - 1)] for e in evb]).mean(axis=0)
    for e in evb:
        e.close()

    # dominant kernel: the gate_up grouped GEMM (2/3 of the flops, 2/3 of the weight bytes)
    gu_s = float(gu_ms.mean()) * 1e-3
    rows = T * (L.E if dense else L.top_k)
    decode_shaped = rows <= 16 * min(L.E, rows) or case.act_dtype == "f32"
    if decode_shaped:
        byts = expert_gemm_bytes(case, 0, n_active, dense)
        achieved = byts / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK["hbm_GBps"], "unit": "GB/s",
                "frac": achieved / PEAK["hbm_GBps"]}
        algo = f"{byts} B per launch ({n_active} routed experts)"
    else:
        fl = expert_gemm_flops(case, 0, dense)
        peak = PEAK["fp8_TFLOPs"] if case.fp8 else PEAK["bf16_TFLOPs"]
        achieved = fl / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak}
        algo = f"{fl} flop per launch"
    roof["kernel"] = gate_up_kernel_name(case, decode_shaped, args.layout == "tiled", dense)
    roof["launches_timed"] = f"{len(gu_ms)} of the {args.steps} timed eager steps (every {EV_EVERY}th)"
    roof["algorithmic"] = algo
    roof["traffic"] = measured_traffic(args.workload, roof["kernel"]) if not dense else None
    res = {
        "metric": METRIC,
        "value": T * args.steps / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x mxfp4" if case.fp8 else case.act_dtype,
        "data": "synthetic (seeded random MXFP4 weights and activations of the named shapes)",
        "config": {"workload": case.name, "E": L.E, "top_k": L.top_k, "H": L.H, "I": L.I, "T": T,
                   "act": "fp8" if case.fp8 else case.act_dtype, "weight_layout": args.layout,
                   "weight_copies": copies,
                   "expert_path": args.path,
                   "routed_experts": n_active,
                   "launch": (f"hip_graph ({GRAPH_STEPS} forwards per graph)" if args.launch == "graph"
                              else "eager (one library call per forward)")},
        "roofline": roof,
        "stages_us": {name: float(v * 1e3) for name, v in zip(STAGES, avg)},
        "stages_note": "separate untimed pass with all stage events (each record adds a few us)",
    }
    if args.launch == "graph":
        res["eager"] = eager
    if decode_shaped and not dense:
        # the whole step against HBM: its algorithmic bytes over the wall
        # time per step (launch gaps and the small stages included)
        sb = step_bytes(case, n_active)
        res["step_hbm"] = {"bytes": sb, "GBps": sb / (ms_step * 1e-3) / 1e9,
                           "frac": sb / (ms_step * 1e-3) / 1e9 / PEAK["hbm_GBps"]}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_budget, dense)
    return res


def bench_unpack(args, dev):
    import torch

    import mxfp4_quantized_moe_amd as mx
    import workloads as W

    case = W.unpack_20b()
    tens = [(W.array_to_torch(b, dev), W.array_to_torch(s, dev)) for b, s in case.tensors]
    outs = [torch.empty(b.shape[:-2] + (b.shape[-2] * 32,), dtype=torch.bfloat16, device=dev) for b, _ in tens]
    byts = sum(b.numel() + s.numel() + o.numel() * 2 for (b, s), o in zip(tens, outs))
    # the plain 256 MiB copy that scales the HBM byte counters of a profiled run
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    torch.empty_like(src).copy_(src)
    del src
    for _ in range(args.warmup):
        for (b, s), o in zip(tens, outs):
            mx.mxfp4_unpack(b, s, out=o)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for (b, s), o in zip(tens, outs):
            mx.mxfp4_unpack(b, s, out=o)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gbps = byts * args.steps / (t1 - t0) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O

        b0, s0 = case.tensors[0]
        rb, rs = b0.reshape(-1, b0.shape[-2], 16), s0.reshape(-1, s0.shape[-1])
        row_bytes = rb.shape[1] * 16 + rb.shape[1] + rb.shape[1] * 32 * 2
        r = oracle_slices(lambda lo, hi: O.mxfp4_unpack(rb[lo:hi], rs[lo:hi]), rb.shape[0], args.cpu_budget,
                          "gate_up rows")
        cpu = {"value": r["rows_per_s"] * row_bytes / 1e9, "unit": "GB/s", "cores": r["cores"], "kind": "oracle",
               "sample": r["sample"]}
    return {"metric": "mxfp4_unpack GB/s (bf16 out)", "value": gbps, "unit": "GB/s", "n_gpus": 1, "cpu_baseline": cpu,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": (t1 - t0) * 1e3 / args.steps,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8->bf16",
            "data": "synthetic", "config": {"workload": case.name, "bytes_per_step": byts},
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK["hbm_GBps"], "unit": "GB/s",
                         "frac": gbps / PEAK["hbm_GBps"], "kernel": "mxmoe::unpack_bf16_kernel",
                         "traffic": measured_traffic("unpack_20b", "mxmoe::unpack_bf16_kernel"),
                         "traffic_unit": "HBM bytes per step (its 2 launches)"}}


def bench_linear(args, dev):
    """The weight-only MXFP4 dense layer: tokens/s and the GEMM's TFLOP/s
    (HIP events around each call on the stream it runs on)."""
    import numpy as np
    import torch

    import mxfp4_quantized_moe_amd as mx
    import workloads as W

    T, K, N = 4096, 2880, 5760
    case = W.linear_case(0, T, K, N, "bf16", True)
    lin = mx.MXFP4Linear(W.array_to_torch(case.blocks, dev), W.array_to_torch(case.scales, dev), N, K,
                         W.array_to_torch(case.bias, dev))
    if args.layout == "tiled":
        lin = lin.tiled()
    wbytes = lin.blocks.numel() + lin.scales.numel()
    copies = min(64, -(-int(1.0e9) // wbytes) + 1) if args.copies is None else args.copies
    lins = [lin] + [mx.MXFP4Linear(lin.blocks.clone(), lin.scales.clone(), N, K, lin.bias, lin.layout)
                    for _ in range(copies - 1)]
    x = W.array_to_torch(case.x, dev)
    out = torch.empty((T, N), dtype=x.dtype, device=dev)
    ws = torch.empty(max(mx.mxfp4_linear_workspace_bytes(T, N, x.dtype), 256), dtype=torch.uint8, device=dev)
    for i in range(args.warmup):
        lins[i % copies](x, out=out, workspace=ws)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record()
        lins[i % copies](x, out=out, workspace=ws)
        ends[i].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    call_s = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)])) * 1e-3
    fl = 2 * T * K * N
    achieved = fl / call_s / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O

        r = oracle_slices(lambda lo, hi: O.mxfp4_linear(case.x[lo:hi], case.blocks, case.scales, case.bias, "bf16"),
                          T, args.cpu_budget, "tokens")
        cpu = {"value": r["rows_per_s"], "unit": "tokens/s", "cores": r["cores"], "kind": "oracle",
               "sample": r["sample"]}
    return {"metric": "MXFP4 dense linear tokens/s", "value": T * args.steps / (t1 - t0), "unit": "tokens/s",
            "cpu_baseline": cpu,
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": (t1 - t0) * 1e3 / args.steps,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded random MXFP4 weight and bf16 activations)",
            "config": {"workload": f"linear_t{T}_k{K}_n{N}", "T": T, "K": K, "N": N, "weight_layout": args.layout,
                       "weight_copies": copies},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK["bf16_TFLOPs"], "unit": "TFLOP/s",
                         "frac": achieved / PEAK["bf16_TFLOPs"], "kernel": "gemm_prefill_tiled_kernel<phase 1>",
                         "algorithmic": f"{fl} flop per call", "traffic": None}}


def bench_fp8_linear(args, dev):
    """The dense FP8 E4M3 layer (W8A8, static per-tensor scales): tokens/s
    and TFLOP/s of the whole call (setup, x quantisation and the GEMM; HIP
    events on the stream it runs on)."""
    import numpy as np
    import torch

    import mxfp4_quantized_moe_amd as mx
    import workloads as W

    T, K, N = 4096, 2880, 5760
    case = W.fp8_linear_case(0, T, K, N)
    lin = mx.FP8Linear.from_codes(W.array_to_torch(case.w_codes, dev), case.w_scale, case.x_scale,
                                  W.array_to_torch(case.bias, dev))
    wbytes = lin.w_tiled.numel()
    copies = min(64, -(-int(1.0e9) // wbytes) + 1) if args.copies is None else args.copies
    lins = [lin] + [mx.FP8Linear(lin.w_tiled.clone(), N, K, lin.w_scale, lin.x_scale, lin.bias)
                    for _ in range(copies - 1)]
    x = W.array_to_torch(case.x, dev)
    out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(mx.fp8_linear_workspace_bytes(T, K, N), 256), dtype=torch.uint8, device=dev)
    for i in range(args.warmup):
        lins[i % copies](x, out=out, workspace=ws)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record()
        lins[i % copies](x, out=out, workspace=ws)
        ends[i].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    call_s = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)])) * 1e-3
    fl = 2 * T * K * N
    achieved = fl / call_s / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O

        r = oracle_slices(lambda lo, hi: O.fp8_linear(case.x[lo:hi], case.w_codes, case.w_scale, case.x_scale,
                                                      case.bias), T, args.cpu_budget, "tokens")
        cpu = {"value": r["rows_per_s"], "unit": "tokens/s", "cores": r["cores"], "kind": "oracle",
               "sample": r["sample"]}
    return {"metric": "FP8 W8A8 dense linear tokens/s", "value": T * args.steps / (t1 - t0), "unit": "tokens/s",
            "cpu_baseline": cpu,
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": (t1 - t0) * 1e3 / args.steps,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
            "data": "synthetic (seeded random e4m3 weight codes and bf16 activations, fixed static scales)",
            "config": {"workload": f"fp8_linear_t{T}_k{K}_n{N}", "T": T, "K": K, "N": N, "weight_copies": copies},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK["fp8_TFLOPs"], "unit": "TFLOP/s",
                         "frac": achieved / PEAK["fp8_TFLOPs"],
                         "kernel": "whole call: setup + x quantisation + gemm_prefill_tiled_kernel<W8A8, phase 1>",
                         "algorithmic": f"{fl} flop per call", "traffic": None}}


def bench_int8(args, dev):
    """The INT8 W8A8 MoE layer at the 20b shape: tokens/s of whole forwards,
    and against the roofline over the forward's duration (HIP events around
    each call on its stream): the two grouped GEMMs' int8 ops against the
    dense int8 peak for a prefill batch, the routed experts' int8 weights
    and scales against HBM for a decode batch."""
    import numpy as np
    import torch

    import mxfp4_quantized_moe_amd as mx
    import workloads as W

    T = int(args.workload.rsplit("t", 1)[1])
    case = W.int8_20b(T)
    L = case.layer
    w0 = W.int8_layer_to_torch(L, dev)
    x = W.array_to_torch(case.x, dev)
    wbytes = w0.gate_up_w.numel() + w0.down_w.numel()
    copies = min(16, -(-int(1.0e9) // wbytes) + 1) if args.copies is None else args.copies
    layers = [w0] + [mx.MoEInt8Weights(w0.gate_up_w.clone(), w0.gate_up_scale, w0.gate_up_bias, w0.down_w.clone(),
                                       w0.down_scale, w0.down_bias, w0.router_w, w0.router_b, w0.top_k)
                     for _ in range(copies - 1)]
    out = torch.empty_like(x)
    ws = torch.empty(max(mx.moe_int8_workspace_bytes(w0, T), 256), dtype=torch.uint8, device=dev)
    idx = torch.empty((T, L.top_k), dtype=torch.int32, device=dev)
    mx.moe_int8_forward(w0, x, out=out, workspace=ws, topk_idx_out=idx)
    n_active = len(np.unique(W.torch_to_array(idx)))
    for i in range(args.warmup):
        mx.moe_int8_forward(layers[i % copies], x, out=out, workspace=ws)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record()
        mx.moe_int8_forward(layers[i % copies], x, out=out, workspace=ws)
        ends[i].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    call_s = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)])) * 1e-3
    ops = 2 * T * L.top_k * (2 * L.I * L.H + L.H * L.I)
    rows = T * L.top_k
    if rows <= 16 * min(L.E, rows):
        # decode-shaped: the routed experts' int8 codes, fp32 row scales and
        # bf16 biases of both matrices, x in and out
        byts = n_active * (3 * L.I * L.H + (2 * L.I + L.H) * (4 + 2)) + 2 * T * L.H * 2
        achieved = byts / call_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK["hbm_GBps"], "unit": "GB/s",
                "frac": achieved / PEAK["hbm_GBps"],
                "algorithmic": f"{byts} B per forward ({n_active} routed experts)"}
    else:
        achieved = ops / call_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK["int8_TOPs"], "unit": "TOP/s",
                "frac": achieved / PEAK["int8_TOPs"], "algorithmic": f"{ops} int8 ops per forward (gate_up + down)"}
    roof.update({"kernel": "whole forward: routing, int8 quantisation of x and h, both grouped GEMMs, combine",
                 "traffic": None})
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O

        r = oracle_slices(lambda lo, hi: O.moe_forward_int8(L, case.x[lo:hi]), T, args.cpu_budget, "tokens")
        cpu = {"value": r["rows_per_s"], "unit": "tokens/s", "cores": r["cores"], "kind": "oracle",
               "sample": r["sample"]}
    return {"metric": "INT8 W8A8 MoE layer tokens/s", "value": T * args.steps / (t1 - t0), "unit": "tokens/s",
            "cpu_baseline": cpu,
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": (t1 - t0) * 1e3 / args.steps,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
            "data": "synthetic (seeded random int8 codes, per-row scales, bf16 activations)",
            "config": {"workload": f"int8_20b_t{T}", "E": L.E, "top_k": L.top_k, "H": L.H, "I": L.I, "T": T,
                       "weight_copies": copies, "routed_experts": n_active},
            "roofline": roof}


# The library's rule for a persistent tiled prefill launch (moe_gemm.hip):
# at least PERSIST_MIN item records per workgroup of the PERSIST_BLOCKS.
PERSIST_MIN, PERSIST_BLOCKS, TILED_ROWS, TILE_TOKENS = 4, 512, 256, 128


def prefill_persistent(case, R: int) -> bool:
    """Whether the routed, tiled prefill GEMM over R weight rows runs as a
    persistent launch (its record grid: max token tiles x row stripes)."""
    rows = case.T * case.layer.top_k
    max_tiles = -(-rows // TILE_TOKENS) + min(rows, case.layer.E)
    blocks = -(-(max_tiles * -(-R // TILED_ROWS)) // 8) * 8
    return blocks >= PERSIST_MIN * PERSIST_BLOCKS


def gate_up_kernel_name(case, decode_shaped: bool, tiled: bool, dense: bool = False) -> str:
    """The gate_up kernel the library launches for this case, as rocprofv3
    names it (template arguments: activation code, phase, then token
    sub-tiles per pass (decode, tiled), persistent launch (prefill, tiled)
    or tiled (row order))."""
    act = 2 if case.fp8 else (1 if case.act_dtype == "bf16" else 0)
    if decode_shaped:
        if tiled and act != 0:
            return f"mxmoe::gemm_decode_tiled_kernel<{act}, 0, {1 if case.T <= 64 else 2}>"
        return f"mxmoe::gemm_decode_kernel<{act}, 0, {'true' if tiled else 'false'}>"
    if tiled:
        persist = not dense and prefill_persistent(case, 2 * case.layer.I)
        return f"mxmoe::gemm_prefill_tiled_kernel<{act}, 0, {'true' if persist else 'false'}>"
    return f"mxmoe::gemm_prefill_kernel<{act}, 0, false>"


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on this kernel and the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        ent = t.get(workload)
        if ent and ent.get("kernel") == kernel and ent.get("kernel_source_hash") == kernel_source_hash():
            return ent["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_120b_t4096")
    ap.add_argument("--copies", type=int, default=None, help="weight copies cycled through (default: >= 1 GB apart)")
    ap.add_argument("--layout", choices=("tiled", "rows"), default="tiled",
                    help="expert weight order: tiled by mxfp4_tile at load (default) or the checkpoint row order")
    ap.add_argument("--path", choices=("routed", "dense"), default="routed",
                    help="experts per token: the routed top_k, or all of them (dense all-experts path)")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="forwards replayed from HIP graphs (default) or one library call each")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures the MoE layer on one MI355X only; runs over several GPUs "
                                   "(expert-parallel sharding) are not implemented", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.steps < 1:
        raise SystemExit("--steps must be >= 1")

    import torch

    import mxfp4_quantized_moe_amd as mx

    mx.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    if args.workload == "unpack_20b":
        res = bench_unpack(args, dev)
    elif args.workload == "linear_t4096_k2880_n5760":
        res = bench_linear(args, dev)
    elif args.workload == "fp8_linear_t4096_k2880_n5760":
        res = bench_fp8_linear(args, dev)
    elif args.workload.startswith("int8_20b_t"):
        res = bench_int8(args, dev)
    else:
        res = bench_layer(args, dev)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
