#!/usr/bin/env python3
"""Throughput of the NVFP4 weight-only Gemma-4-26B-A4B MoE expert block on one
MI355X.

A step is one pass of the whole hot path -- routing, bucketing and the expert
input's prep (one moe_route_bucket_prep call), the expert MLP's gate/up and
down projections, and moe_combine -- over one batch of seeded synthetic tokens,
with inputs and weights already resident in HBM.  The default workload is one
model-shaped layer at decode batch T = 64 (hidden 2816, 128 experts, top-8,
expert intermediate 704, NVFP4 experts from bf16 N(0, 0.02)).

Timing: W warm-up steps, then K steps captured in one HIP graph on one stream
and replayed once, bracketed by synchronisations (ms_per_step is wall clock /
K).  The dominant kernel (the gate/up GEMV/GEMM) is timed by HIP events around
back-to-back launches of its stage call on the same stream; per-stage
durations come from a second graph of the K steps in which every stage call is
a child graph between timing-event nodes.  Consecutive steps read different,
byte-identical copies of the expert weights so that each step streams its
experts from HBM instead of the 256 MB last-level cache.

Prints one JSON line (rank 0).
"""
import argparse
import ctypes
import json
import math
import os
import re
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense f16/bf16 MFMA
STAGES = ("route_bucket_prep", "gate_up", "down", "combine")
SEPARATE_STAGES = ("route_bucket", "prep", "gate_up", "down", "combine")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200; 10 for the 30-layer sweep)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 20; 3 for the 30-layer sweep)")
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3, 4],
                    help="0: T=4, 1: T=64 (default), 2: T=2048 Zipf, 4: T=16384 Zipf+outliers, "
                         "3: 30-layer decode sweep")
    ap.add_argument("--sweep-T", type=int, default=8, help="tokens per layer for workload 3 (1 or 8)")
    ap.add_argument("--chain", action="store_true",
                    help="workload 3: chain the layers through the residual (each layer's sparse "
                         "branch with its learned norms reads the previous layer's output)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the token count of workload 0, 1, 2 or 4 (a size sweep)")
    ap.add_argument("--replicas", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--format", default="nvfp4", choices=["nvfp4", "q4_0", "aff4"],
                    help="expert weight format (the int4 ones: seeded codes and fp16 scales)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=64,
                    help="tokens of the workload the fp64 oracle baseline runs (about 10-20 s)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--separate-prep", action="store_true",
                    help="queue moe_route_bucket and the expert-input prep as two calls instead "
                         "of one moe_route_bucket_prep")
    ap.add_argument("--prep-branch", action="store_true",
                    help="with --separate-prep: run the prep on a parallel graph branch (forked "
                         "and joined per layer) instead of first on the one stream")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter scaling reference)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 10 if args.workload == 3 else 200
    if args.warmup is None:
        args.warmup = 3 if args.workload == 3 else 20
    return args


class HipRuntime:
    """The few HIP runtime calls torch does not expose on ROCm: timing events
    recorded as external nodes of a captured graph, capture and launch of that
    graph.  Uses the HIP runtime torch has already loaded."""

    def __init__(self):
        path = next((l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l),
                    "libamdhip64.so")
        h = ctypes.CDLL(path)
        vp, P = ctypes.c_void_p, ctypes.POINTER
        for name, args in {"hipEventCreate": [P(vp)], "hipEventRecordWithFlags": [vp, vp, ctypes.c_uint],
                           "hipEventRecord": [vp, vp], "hipStreamWaitEvent": [vp, vp, ctypes.c_uint],
                           "hipEventElapsedTime": [P(ctypes.c_float), vp, vp],
                           "hipStreamBeginCapture": [vp, ctypes.c_int],
                           "hipStreamEndCapture": [vp, P(vp)],
                           "hipGraphInstantiate": [P(vp), vp, vp, ctypes.c_char_p, ctypes.c_size_t],
                           "hipGraphLaunch": [vp, vp], "hipGetErrorString": [ctypes.c_int],
                           "hipGraphCreate": [P(vp), ctypes.c_uint],
                           "hipGraphAddEventRecordNode": [P(vp), vp, P(vp), ctypes.c_size_t, vp],
                           "hipGraphAddChildGraphNode": [P(vp), vp, P(vp), ctypes.c_size_t, vp]}.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "hipGetErrorString" else ctypes.c_int
        self.h = h

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {self.h.hipGetErrorString(rc).decode()}")

    def event(self):
        ev = ctypes.c_void_p()
        self._ok(self.h.hipEventCreate(ctypes.byref(ev)), "hipEventCreate")
        return ev

    def record(self, ev, stream, external):
        if external:
            self._ok(self.h.hipEventRecordWithFlags(ev, stream, 1), "hipEventRecordWithFlags")
        else:
            self._ok(self.h.hipEventRecord(ev, stream), "hipEventRecord")

    def wait(self, stream, ev):
        self._ok(self.h.hipStreamWaitEvent(stream, ev, 0), "hipStreamWaitEvent")

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        self._ok(self.h.hipEventElapsedTime(ctypes.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def capture_graph(self, stream, fn):
        """Stream-capture whatever fn() queues on `stream` into a graph."""
        self._ok(self.h.hipStreamBeginCapture(stream, 2), "hipStreamBeginCapture")  # relaxed
        graph = ctypes.c_void_p()
        try:
            fn()
        finally:
            rc = self.h.hipStreamEndCapture(stream, ctypes.byref(graph))
        self._ok(rc, "hipStreamEndCapture")
        return graph

    def timed_chain(self, stream, calls, events):
        """One graph: event[0], calls[0], event[1], calls[1], ... event[n] as a
        chain of event-record nodes and child-graph nodes (each call captured
        into its own child graph)."""
        g = ctypes.c_void_p()
        self._ok(self.h.hipGraphCreate(ctypes.byref(g), 0), "hipGraphCreate")
        prev = None

        def add_event(ev):
            node = ctypes.c_void_p()
            deps = (ctypes.c_void_p * 1)(prev) if prev is not None else None
            self._ok(self.h.hipGraphAddEventRecordNode(ctypes.byref(node), g, deps,
                                                       0 if prev is None else 1, ev),
                     "hipGraphAddEventRecordNode")
            return node

        prev = add_event(events[0])
        for call, ev in zip(calls, events[1:]):
            child = self.capture_graph(stream, call)
            node = ctypes.c_void_p()
            deps = (ctypes.c_void_p * 1)(prev)
            self._ok(self.h.hipGraphAddChildGraphNode(ctypes.byref(node), g, deps, 1, child),
                     "hipGraphAddChildGraphNode")
            prev = node
            prev = add_event(ev)
        return self.instantiate(g)

    def instantiate(self, g):
        exe = ctypes.c_void_p()
        self._ok(self.h.hipGraphInstantiate(ctypes.byref(exe), g, None, None, 0),
                 "hipGraphInstantiate")
        return exe

    def launch(self, exe, stream):
        self._ok(self.h.hipGraphLaunch(exe, stream), "hipGraphLaunch")


# scale bytes per 32 weights: two E4M3 codes (NVFP4), one fp16 d (q4_0), fp16 s and b (aff4)
SCALE_BYTES_PER_32 = {"nvfp4": 2, "q4_0": 2, "aff4": 4}
FORMAT_INDEX = {"nvfp4": 0, "q4_0": 1, "aff4": 2}


def proj_bytes(H, I, fmt="nvfp4"):
    """Bytes of one expert's [I, H] (or [H, I]) projection: packed nibbles,
    block scales, and the FP32 tensor scale of NVFP4."""
    return H * I // 2 + H * I * SCALE_BYTES_PER_32[fmt] // 32 + (4 if fmt == "nvfp4" else 0)


def expert_bytes_per_expert(H, I, fmt="nvfp4"):
    return 3 * proj_bytes(H, I, fmt)


def main():
    args = parse()
    if args.copy_reference:
        copy_reference(args.copy_reference)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the expert-parallel "
              "multi-GPU path is described, not implemented.", file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_synth as S
    import nvfp4_weight_only_moe_amd as moe
    from nvfp4_weight_only_moe_amd import workload as Wl

    torch.cuda.set_device(0)
    moe.lib()
    wl = dict(S.WORKLOADS[args.workload])
    if args.tokens and args.workload != 3:
        wl["T"] = (args.tokens,)
        wl["name"] = re.sub(r"_T\d+", f"_T{args.tokens}", wl["name"])
    H, I, E, K = S.H, S.I, S.E, S.TOP_K
    t_setup = time.perf_counter()

    fmt = args.format
    if fmt != "nvfp4":
        wl["name"] += f"_{fmt}"

    def make_layer(l, zipf):
        if fmt == "nvfp4":
            return Wl.build_layer(l, zipf=zipf)
        return Wl.build_int4_layer(fmt, l, zipf=zipf)

    if args.workload == 3:
        T = args.sweep_T
        layers = [make_layer(l, False) for l in range(S.LAYERS)]
        step_layers = [layers]                       # one step = the 30-layer sweep
        replicas = 1                                 # 12.85 GB of distinct weights per sweep
    else:
        T = wl["T"][0]
        base = make_layer(0, wl["zipf"])
        touched = expert_bytes_per_expert(H, I, fmt) * min(E, T * K)
        replicas = args.replicas or max(2, min(16, math.ceil(1.5 * 2 ** 30 / touched) + 1))
        reps = Wl.replicate_experts(base, replicas)
        step_layers = [[r] for r in reps]
    x = Wl.to_device_bf16(S.activations(args.workload, T, outliers=wl["outliers"]))
    buf = moe.MoeBuffers(T, H, I, E, K)
    # chained sweep: layer l reads xs[l] and writes xs[l + 1] (xs[0] = x, so
    # every step runs the same chain)
    chain = args.chain and args.workload == 3
    if chain:
        wl["name"] += "_chained"
        norms = [moe.BranchNorms(*[Wl.to_device_bf16(a) for a in S.norm_weights(l)])
                 for l in range(len(step_layers[0]))]
        xs = [x] + [torch.empty_like(x) for _ in step_layers[0]]
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup

    def one_step(s, marks=None):
        for li, layer in enumerate(step_layers[s % len(step_layers)]):
            if chain:
                moe.forward_branch(layer, xs[li], buf, norms[li])
                xs[li + 1].copy_(buf.out)
            else:
                moe.forward(layer, x, buf, marks=marks)

    for s in range(args.warmup):
        one_step(s)
    torch.cuda.synchronize()

    # K steps, a timing event around every stage call.  With a graph the
    # events are external event-record nodes of the graph itself.
    n_layers = len(step_layers[0])
    hip = HipRuntime()
    stream, side = torch.cuda.Stream(), torch.cuda.Stream()
    hs, hside = ctypes.c_void_p(stream.cuda_stream), ctypes.c_void_p(side.cuda_stream)
    from nvfp4_weight_only_moe_amd import _lib as C

    separate = args.separate_prep or args.prep_branch
    stages = SEPARATE_STAGES if separate else STAGES

    def stage_calls(layer, prep_stream=None, li=0):
        """The stage calls of one block pass (layer li of the step), by name."""
        x_in = xs[li] if chain else x
        nm = norms[li] if chain else None
        if chain:
            prep = lambda: C.nvfp4_expert_prep_rmsnorm(x_in, nm.pre, nm.eps, E, I, K, buf.ws,
                                                       prep_stream or stream)
            combine = lambda: C.moe_combine_rmsnorm(buf.y_sorted, buf.topk_w, buf.pair_rank,
                                                    nm.post, nm.eps, xs[li + 1], x_in,
                                                    nm.layer_scalar, stream)
        else:
            prep = lambda: C.nvfp4_expert_prep(x_in, E, I, K, buf.ws, prep_stream or stream)
            combine = lambda: C.moe_combine(buf.y_sorted, buf.topk_w, buf.pair_rank, buf.out,
                                            stream)
        return {
            "route_bucket_prep": lambda: C.moe_route_bucket_prep(
                x_in, layer.w_router, layer.router_scale, layer.per_expert_scale,
                layer.logit_bias, K, layer.eps, buf.topk_idx, buf.topk_w, buf.topk_w_raw,
                buf.logits, buf.expert_offsets, buf.sorted_pairs, buf.pair_rank, buf.bucket_ws,
                nm.pre if chain else None, nm.eps if chain else 0.0, I, buf.ws, stream),
            "route_bucket": lambda: C.moe_route_bucket(
                x_in, layer.w_router, layer.router_scale, layer.per_expert_scale,
                layer.logit_bias, K, layer.eps, buf.topk_idx, buf.topk_w, buf.topk_w_raw,
                buf.logits, buf.expert_offsets, buf.sorted_pairs, buf.pair_rank, buf.bucket_ws,
                stream),
            "prep": prep,
            "gate_up": lambda: C.nvfp4_expert_gate_up(layer.gate, layer.up, buf.expert_offsets,
                                                      buf.sorted_pairs, T, K, H, buf.ws, stream),
            "down": lambda: C.nvfp4_expert_down(layer.down, buf.expert_offsets, T, K,
                                                buf.y_sorted, buf.ws, stream),
            "combine": combine,
        }

    step_plan = [step_layers[(args.warmup + s) % len(step_layers)] for s in range(args.steps)]
    fork_join = [(hip.event(), hip.event()) for _ in range(args.steps * n_layers)]

    def queue_steps():
        """K steps on one stream: per layer route + bucket + prep (one call),
        gate/up, down, combine.  --separate-prep: prep, then route + bucket,
        as two calls; --prep-branch: the prep on `side` instead, forked after
        the previous layer's combine and joined before the gate/up GEMM (a
        dependency across queues costs more than the prep)."""
        n = 0
        for layers in step_plan:
            for li, layer in enumerate(layers):
                c = stage_calls(layer, side if args.prep_branch else None, li)
                if args.prep_branch:
                    fork, join = fork_join[n]
                    n += 1
                    hip.record(fork, hs, False)
                    hip.wait(hside, fork)
                    c["prep"]()
                    hip.record(join, hside, False)
                    c["route_bucket"]()
                    hip.wait(hs, join)
                elif separate:
                    c["prep"]()
                    c["route_bucket"]()
                else:
                    c["route_bucket_prep"]()
                c["gate_up"]()
                c["down"]()
                c["combine"]()

    # ---- timed region: the K steps as one graph, replayed once
    mode, graph = "eager", None
    torch.cuda.synchronize()
    if not args.eager:
        try:
            graph = hip.instantiate(hip.capture_graph(hs, queue_steps))
            mode = ("hip_graph (prep on a parallel branch)" if args.prep_branch else
                    "hip_graph (one stream, route + prep as two calls)" if separate else
                    "hip_graph (one stream)")
            hip.launch(graph, hs)            # one untimed replay
            stream.synchronize()
        except Exception as exc:
            print(f"graph build failed ({exc}); timing eager launches", file=sys.stderr)
            graph = None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        hip.launch(graph, hs)
    else:
        queue_steps()
    stream.synchronize()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # ---- per-stage durations: the same K steps with every stage call a
    # child graph between timing-event nodes (serial order, one stream)
    calls = []
    for layers in step_plan:
        for li, layer in enumerate(layers):
            c = stage_calls(layer, None, li)
            calls += [c[n] for n in stages]
    bounds = [hip.event() for _ in range(len(calls) + 1)]   # event i precedes call i
    if not args.eager:
        timed_graph = hip.timed_chain(hs, calls, bounds)
        hip.launch(timed_graph, hs)
        events_mode = "hip_graph_with_event_nodes"
    else:
        hip.record(bounds[0], hs, False)
        for call, e in zip(calls, bounds[1:]):
            call()
            hip.record(e, hs, False)
        events_mode = "eager_with_events"
    stream.synchronize()
    torch.cuda.synchronize()

    # ---- the dominant kernel alone: the gate/up stage call R times back to
    # back (the same routing and buffers, the layers of the step plan in
    # turn, so the weights stream from HBM as in the steps) between two
    # timing events on the launch stream; the event cost spreads over R
    gu_calls = [stage_calls(layers[li], None, li)["gate_up"]
                for layers in step_plan for li in range(len(layers))]
    reps_gu = max(20, len(gu_calls))
    gu_seq = [gu_calls[i % len(gu_calls)] for i in range(reps_gu)]
    gu_ev = [hip.event(), hip.event()]
    if not args.eager:
        gu_graph = hip.timed_chain(hs, [lambda: [c() for c in gu_seq]], gu_ev)
        hip.launch(gu_graph, hs)                    # warm
        stream.synchronize()
        hip.launch(gu_graph, hs)
    else:
        hip.record(gu_ev[0], hs, False)
        for c in gu_seq:
            c()
        hip.record(gu_ev[1], hs, False)
    stream.synchronize()
    gu_kernel_us = 1e3 * hip.elapsed(gu_ev[0], gu_ev[1]) / reps_gu

    stage_ms = {n: [] for n in stages}
    gpu_step_ms = []
    per_step = n_layers * len(stages)
    for s in range(args.steps):
        b = bounds[s * per_step:(s + 1) * per_step + 1]
        for j in range(per_step):
            stage_ms[stages[j % len(stages)]].append(hip.elapsed(b[j], b[j + 1]))
        gpu_step_ms.append(hip.elapsed(b[0], b[-1]))
    stage_avg_us = {n: 1e3 * float(np.mean(v)) for n, v in stage_ms.items()}

    # work done per step (realised routing)
    counts = np.diff(buf.expert_offsets.cpu().numpy())
    U = int((counts > 0).sum())                  # active experts of the last layer run
    P = T * K
    if args.workload == 3:
        U_layers = []
        for li, layer in enumerate(step_layers[0]):
            if chain:
                moe.forward_branch(layer, xs[li], buf, norms[li])
                xs[li + 1].copy_(buf.out)
            else:
                moe.forward(layer, x, buf)
            torch.cuda.synchronize()
            U_layers.append(int((np.diff(buf.expert_offsets.cpu().numpy()) > 0).sum()))
        U_total = sum(U_layers)
    else:
        U_layers, U_total = [U], U
    per_exp = expert_bytes_per_expert(H, I, fmt)
    gu_w_bytes = 2 * proj_bytes(H, I, fmt)
    step_s = ms_per_step / 1e3
    # the back-to-back gate/up launches all ran on the routing still in buf
    # (the last layer queued before them), whose U is counted above
    gate_up_alg_bytes = gu_w_bytes * U + T * H * 2 + P * I * 2     # per launch
    gu_us = gu_kernel_us
    achieved_gbps = gate_up_alg_bytes / (gu_us * 1e-6) / 1e9
    expert_flops = 2.0 * P * 3 * I * H * n_layers
    out = {
        "metric": "MoE layer tokens/s; decode NVFP4 weight GB/s; prefill TFLOP/s (1 MI355X)",
        "value": T / step_s if args.workload != 3 else T / step_s,
        "unit": "tokens/s" if args.workload != 3 else "tokens/s (30-layer sweep)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[fmt] + " x bf16 activations; f16 MFMA, fp32 accumulate",
        "data": DATA[fmt],
        "config": {"workload": wl["name"], "tokens": T, "hidden": H, "experts": E, "top_k": K,
                   "moe_intermediate": I, "layers": n_layers, "weight_replicas": replicas,
                   "timing": mode},
        "detail": {
            "stage_timing": events_mode,
            "chained_layers": bool(chain),
            "gpu_ms_per_step_with_event_nodes": float(np.mean(gpu_step_ms)),
            "stage_avg_us": stage_avg_us,
            "gate_up_kernel_us_back_to_back": gu_kernel_us,
            "active_experts": U_total,
            "expert_weight_GBps": per_exp * U_total / step_s / 1e9,
            "layer_alg_GBps": (per_exp * U_total + n_layers * ((E * H + H + E) * 2 + 2 * T * H * 2)) / step_s / 1e9,
            "expert_TFLOPs": expert_flops / step_s / 1e12,
            "max_over_mean_bucket": float(counts.max() / max(counts.mean(), 1e-9)),
            "setup_s": t_setup,
        },
    }
    # Roofline of the dominant kernel, the gate/up projection: the HBM one for
    # decode (its algorithmic bytes: the active experts' gate and up tensors,
    # the f16 activations and A written), the f16 MFMA one for prefill (its
    # algorithmic flops 2 P 2 I H); the other one is reported beside it.
    gu_kernel = gate_up_kernel_name(T, K, E, fmt)
    traffic = profiled_traffic(wl["name"], gu_kernel)   # HBM bytes per launch (counters)
    hbm = {"kernel": gu_kernel, "bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS,
           "unit": "GB/s", "frac": achieved_gbps / HBM_PEAK_GBPS, "traffic": traffic,
           "alg_bytes_per_launch": gate_up_alg_bytes, "avg_launch_us": gu_us,
           "units": f"{U} active experts x {gu_w_bytes} B + {T} x {H} x 2 B + {P} x {I} x 2 B"}
    gu_flops = 2.0 * P * 2 * I * H
    tflops = gu_flops / (gu_us * 1e-6) / 1e12
    mfma = {"kernel": gu_kernel, "bound": "mfma", "achieved": tflops, "peak": F16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": tflops / F16_MFMA_PEAK_TFLOPS, "traffic": traffic,
            "alg_flops_per_launch": gu_flops, "avg_launch_us": gu_us}
    if args.workload in (2, 4):
        out["roofline"], out["roofline_hbm"] = mfma, hbm
    else:
        out["roofline"], out["roofline_mfma"] = hbm, mfma
    if not args.no_cpu_baseline and args.workload != 3:
        out["cpu_baseline"] = cpu_baseline(args, wl, T)
    print(json.dumps(out), flush=True)


S_I = 704  # expert intermediate size of the workloads
DTYPES = {"nvfp4": "nvfp4 weights (e2m1 x e4m3 x fp32)",
          "q4_0": "int4 q4_0 weights ((q - 8) x fp16 d per 32)",
          "aff4": "int4 affine weights (q x fp16 s + fp16 b per 32)"}
DATA = {"nvfp4": "synthetic (seeded; bf16 N(0,0.02) experts quantised to NVFP4 on the GPU)",
        "q4_0": "synthetic (seeded; uniform int4 codes, fp16 d ~ U(0.004, 0.008))",
        "aff4": "synthetic (seeded; uniform int4 codes, fp16 s ~ U(0.004, 0.008), "
                "b ~ U(-0.06, -0.035))"}


def gate_up_kernel_name(T, K, E, fmt="nvfp4"):
    """The kernel nvfp4_expert_gate_up launches for this shape (the dispatch
    rule of the library: few rows per expert -> GEMV mode)."""
    P = T * K
    avg = P // max(1, min(P, E))
    f = FORMAT_INDEX[fmt]
    if avg < 24:
        rows = 8 if P <= 4 * E else 16
        return f"k_expert_gemv<{rows}, 2, true, 4, {f}>"
    return f"k_expert_gemm<4, 2, true, {f}>"


def profiled_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of this workload, or None when there is none or when the kernel
    source has changed since the counters were taken (the summary records
    the sha256 of mlp.hip followed by common.h as they were then)."""
    import hashlib
    path = os.path.join(HERE, "profiles", f"hbm_traffic__{workload}.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in ("mlp.hip", "common.h"):     # the expert kernels and their decode
        h.update(open(os.path.join(HERE, "nvfp4_weight_only_moe_amd", "csrc", f), "rb").read())
    digest = h.hexdigest()
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != digest or rec.get("kernel") != kernel:
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_reference(mib):
    """A plain device-to-device copy of `mib` MiB (three launches), the
    reference that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to
    bytes: each launch reads and writes exactly mib MiB."""
    import torch
    torch.cuda.set_device(0)
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes_per_launch": n, "launches": 3}), flush=True)


def cpu_baseline(args, wl, T):
    """The fp64 oracle as it stands, single-threaded, on a bounded sample of
    the same workload: the block for the first n tokens (expert weights
    quantised by the oracle itself beforehand, untimed)."""
    from threadpoolctl import threadpool_limits
    import moe_synth as S
    from oracle import formats as F
    from oracle import int4 as Q
    from oracle import moe as M
    from oracle.quantize import quantize
    from concurrent.futures import ThreadPoolExecutor

    n = min(T, args.cpu_sample_tokens)
    p = S.router_params(0, zipf=wl["zipf"])
    r = dict(w_router=F.bf16_bits_to_f64(p["w_router"]), scale=F.bf16_bits_to_f64(p["scale"]),
             per_expert_scale=F.bf16_bits_to_f64(p["per_expert_scale"]), bias=p["bias"])
    x = F.bf16_bits_to_f64(S.activations(args.workload, T, outliers=wl["outliers"]))[:n]
    ids = M.route(x, r["w_router"], r["scale"], r["per_expert_scale"], 8, r["bias"])["idx"]
    todo = [(proj, int(e)) for e in np.unique(ids) for proj in (S.GATE, S.UP, S.DOWN)]

    fmt = args.format

    def q(item):
        proj, e = item
        if fmt != "nvfp4":
            return item, S.int4_expert(fmt, 0, proj, e)
        return item, quantize(F.bf16_bits_to_f64(S.expert_weight(0, proj, e)))

    with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        packed = dict(ex.map(q, todo))                    # weight preparation, untimed

    def decode(item):
        if fmt == "nvfp4":
            return F.dequantize(*packed[item])
        p, sb = packed[item]
        bits = sb.view(np.uint16)
        if fmt == "q4_0":
            return Q.decode_q4_0(p, bits)
        return Q.decode_aff4(p, bits.reshape(bits.shape[0], -1, 2))
    fn = {proj: (lambda e, proj=proj: decode((proj, e))) for proj in (S.GATE, S.UP, S.DOWN)}
    # the same block again until at least 10 s have been timed (the expert
    # decode, not the token count, dominates one run)
    runs, dt = 0, 0.0
    with threadpool_limits(1):
        while runs == 0 or (dt < 10.0 and runs < 8):
            t0 = time.perf_counter()
            M.moe_block(x, x, r, fn[S.GATE], fn[S.UP], fn[S.DOWN], k=8)
            dt += time.perf_counter() - t0
            runs += 1
    return {"value": n * runs / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of the {T} tokens of {wl['name']} through the fp64 oracle block "
                      f"(route, bucket, {fmt} decode of the {len(todo) // 3} touched experts, "
                      f"expert MLPs, combine), {runs} run(s) in {dt:.1f} s"}


if __name__ == "__main__":
    main()
