#!/usr/bin/env python3
"""Throughput of the NVFP4 weight-only Gemma-4-26B-A4B MoE expert block on one
MI355X.

A step is one pass of the whole hot path -- routing, bucketing and the expert
input's prep, the expert MLP's gate/up and down projections, and the weighted
combine -- over one batch of seeded synthetic tokens, with inputs and weights
already resident in HBM.  Model shapes: hidden 2816, 128 experts, top-8,
expert intermediate 704, NVFP4 experts quantised on the GPU from bf16
N(0, 0.02).

Workloads (--workload):
  0  one layer, decode T = 4
  1  one layer, decode T = 64 (the headline line)
  2  one layer, prefill T = 2048, Zipf(1.2) expert popularity
  3  the 30-layer stack (12.85 GB of NVFP4 experts), one decode sweep through
     all 30 layers per step, T = 1 or 8 (--sweep-T)
  4  one layer, prefill T = 16384, Zipf(1.2) + 1% outlier rows x20
Without --workload every one of them is measured: the JSON line is workload
1's, and detail.workloads holds each workload's own figures (T = 1 and T = 8
for workload 3).

Timing: W warm-up steps, then K steps captured in one HIP graph on one stream.
The graph is launched twice back to back; ms_per_step is the GPU time of the
second replay from HIP events recorded on the same stream before and after it,
divided by K, so the host's launch of the graph overlaps the first replay as
it overlaps the previous step in a serving loop.  The first replay's time
(launched onto an idle stream, the GPU waiting for the graph's packets) and
the host wall clock per replay are reported beside it.  The
dominant kernel (the gate/up projection) is timed by HIP events around
back-to-back launches of its stage call on the same stream.  Consecutive steps
of a single-layer workload read different, byte-identical copies of the expert
weights, so that each step streams its experts from HBM instead of the 256 MB
last-level cache.

Prints one JSON line.
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
METRIC = "MoE layer tokens/s; decode NVFP4 weight GB/s; prefill TFLOP/s (1 MI355X)"
# the workloads of the default run, in order: (workload, tokens per layer)
ALL_RUNS = ((1, 64), (0, 4), (2, 2048), (4, 16384), (3, 1), (3, 8))


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200 for one layer, 20 for the 30-layer sweep)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 20 for one layer, 3 for the sweep)")
    ap.add_argument("--workload", type=int, default=None, choices=[0, 1, 2, 3, 4],
                    help="measure one workload only (default: all, workload 1 as the headline)")
    ap.add_argument("--sweep-T", type=int, default=8, help="tokens per layer for workload 3")
    ap.add_argument("--chain", action="store_true",
                    help="workload 3: chain the layers through the residual (each layer's sparse "
                         "branch with its learned norms and the layer step reads the previous "
                         "layer's output)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the token count of workload 0, 1, 2 or 4 (a size sweep)")
    ap.add_argument("--replicas", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--format", default="nvfp4", choices=["nvfp4", "q4_0", "aff4"],
                    help="expert weight format (the int4 ones: seeded codes and fp16 scales)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=64,
                    help="tokens of the workload the fp64 oracle baseline runs")
    ap.add_argument("--stages", action="store_true",
                    help="also time every stage call (a second graph with event nodes)")
    ap.add_argument("--four-calls", action="store_true",
                    help="run decode batches through the separate calls instead of "
                         "moe_layer_decode")
    ap.add_argument("--separate-prep", action="store_true",
                    help="queue moe_route_bucket and the expert-input prep as two calls instead "
                         "of one moe_route_bucket_prep")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter scaling reference)")
    return ap.parse_args(argv)


def step_defaults(workload, steps, warmup):
    sweep = workload == 3
    return (steps if steps is not None else (20 if sweep else 200),
            warmup if warmup is not None else (3 if sweep else 20))


class HipRuntime:
    """The few HIP runtime calls torch does not expose on ROCm: events recorded
    on a raw stream or as nodes of a graph, stream capture, graph launch.
    Uses the HIP runtime torch has already loaded."""

    def __init__(self):
        path = next((l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l),
                    "libamdhip64.so")
        h = ctypes.CDLL(path)
        vp, P = ctypes.c_void_p, ctypes.POINTER
        for name, args in {"hipEventCreate": [P(vp)], "hipEventRecord": [vp, vp],
                           "hipEventElapsedTime": [P(ctypes.c_float), vp, vp],
                           "hipStreamBeginCapture": [vp, ctypes.c_int],
                           "hipStreamEndCapture": [vp, P(vp)],
                           "hipGraphInstantiate": [P(vp), vp, vp, ctypes.c_char_p, ctypes.c_size_t],
                           "hipGraphLaunch": [vp, vp], "hipGetErrorString": [ctypes.c_int],
                           "hipGraphCreate": [P(vp), ctypes.c_uint],
                           "hipGraphExecDestroy": [vp],
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

    def record(self, ev, stream):
        self._ok(self.h.hipEventRecord(ev, stream), "hipEventRecord")

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        self._ok(self.h.hipEventElapsedTime(ctypes.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def capture(self, stream, fn):
        """Stream-capture whatever fn() queues on `stream` into a graph."""
        self._ok(self.h.hipStreamBeginCapture(stream, 2), "hipStreamBeginCapture")  # relaxed
        graph = ctypes.c_void_p()
        try:
            fn()
        finally:
            rc = self.h.hipStreamEndCapture(stream, ctypes.byref(graph))
        self._ok(rc, "hipStreamEndCapture")
        return graph

    def instantiate(self, g):
        exe = ctypes.c_void_p()
        self._ok(self.h.hipGraphInstantiate(ctypes.byref(exe), g, None, None, 0),
                 "hipGraphInstantiate")
        return exe

    def launch(self, exe, stream):
        self._ok(self.h.hipGraphLaunch(exe, stream), "hipGraphLaunch")

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
            child = self.capture(stream, call)
            node = ctypes.c_void_p()
            deps = (ctypes.c_void_p * 1)(prev)
            self._ok(self.h.hipGraphAddChildGraphNode(ctypes.byref(node), g, deps, 1, child),
                     "hipGraphAddChildGraphNode")
            prev = node
            prev = add_event(ev)
        return self.instantiate(g)

    def timed_replay(self, exe, stream, sync):
        """GPU milliseconds of one replay of `exe` in steady state, and of a
        replay launched onto an idle stream, plus the host wall-clock
        milliseconds per replay.  Two replays are queued back to back with
        events before, between and after them: the second one's GPU time
        (between the middle and the last event) excludes the host-side launch
        of the graph, which overlaps the first replay's execution, as it
        overlaps the previous step's in a serving loop; the first one's
        includes it (the GPU waits for the graph's packets)."""
        a, b, c = self.event(), self.event(), self.event()
        sync()
        t0 = time.perf_counter()
        self.record(a, stream)
        self.launch(exe, stream)
        self.record(b, stream)
        self.launch(exe, stream)
        self.record(c, stream)
        sync()
        wall = (time.perf_counter() - t0) * 1e3 / 2
        return self.elapsed(b, c), wall, self.elapsed(a, b)


# scale bytes per 32 weights: two E4M3 codes (NVFP4), one fp16 d (q4_0), fp16 s and b (aff4)
SCALE_BYTES_PER_32 = {"nvfp4": 2, "q4_0": 2, "aff4": 4}
FORMAT_INDEX = {"nvfp4": 0, "q4_0": 1, "aff4": 2}


def proj_bytes(H, I, fmt="nvfp4"):
    """Bytes of one expert's [I, H] (or [H, I]) projection: packed nibbles,
    block scales, and the FP32 tensor scale of NVFP4."""
    return H * I // 2 + H * I * SCALE_BYTES_PER_32[fmt] // 32 + (4 if fmt == "nvfp4" else 0)


def expert_bytes_per_expert(H, I, fmt="nvfp4"):
    return 3 * proj_bytes(H, I, fmt)


def gate_up_kernel_name(T, K, E, fmt="nvfp4"):
    """The kernel nvfp4_expert_gate_up launches for this shape (the dispatch
    rule of the library: few rows per expert -> GEMV mode; 128 or more ->
    128-row GEMM blocks)."""
    P = T * K
    avg = P // max(1, min(P, E))
    f = FORMAT_INDEX[fmt]
    if avg < 24:
        rows = 8 if P <= 4 * E else 16
        return f"k_expert_gemv<{rows}, 2, true, 4, {f}, 1>"   # ..., prefetch depth 1
    return f"k_expert_gemm<{8 if avg >= 128 else 4}, 2, true, {f}>"


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
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != h.hexdigest() or rec.get("kernel") != kernel:
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Bench:
    """Device state shared by the workloads of one run: layer 0's expert
    weights (and their byte-identical replicas) behind either router, the
    30-layer stack when asked for, the HIP runtime and one stream."""

    def __init__(self, args):
        import torch
        import moe_synth as S
        import nvfp4_weight_only_moe_amd as moe
        from nvfp4_weight_only_moe_amd import workload as Wl
        from nvfp4_weight_only_moe_amd import _lib as C
        self.torch, self.S, self.moe, self.Wl, self.C = torch, S, moe, Wl, C
        self.args = args
        self.fmt = args.format
        self.hip = HipRuntime()
        self.stream = torch.cuda.Stream()
        self.hs = ctypes.c_void_p(self.stream.cuda_stream)
        self.H, self.I, self.E, self.K = S.H, S.I, S.E, S.TOP_K
        self._base, self._reps, self._stack = None, [], None

    def make_layer(self, l, zipf):
        if self.fmt == "nvfp4":
            return self.Wl.build_layer(l, zipf=zipf)
        return self.Wl.build_int4_layer(self.fmt, l, zipf=zipf)

    def single_layer(self, zipf, replicas):
        """`replicas` byte-identical copies of layer 0's experts behind the
        plain or the Zipf-biased router."""
        S, Wl, moe = self.S, self.Wl, self.moe
        if self._base is None:
            self._base = self.make_layer(0, False)
            self._reps = [self._base]
        while len(self._reps) < replicas:
            b = self._base
            self._reps.append(b.with_experts(b.gate.clone(), b.up.clone(), b.down.clone()))
        reps = self._reps[:replicas]
        if zipf:
            wr, sc, pes, bias = Wl.router_to_device(S.router_params(0, zipf=True))
            reps = [moe.MoeLayer(wr, sc, pes, bias, r.gate, r.up, r.down, self.K) for r in reps]
        return reps

    def stack(self):
        if self._stack is None:
            self._stack = [self.make_layer(l, False) for l in range(self.S.LAYERS)]
        return self._stack


def run_workload(B, workload, T, steps, warmup, stages=False, chain=False, name=None):
    """Measure one workload: K steps in one graph, replayed once, event-timed;
    the gate/up kernel alone; the work done.  Returns a dict of figures."""
    torch, S, moe, C, hip = B.torch, B.S, B.moe, B.C, B.hip
    H, I, E, K, fmt = B.H, B.I, B.E, B.K, B.fmt
    wl = dict(S.WORKLOADS[workload])
    name = name or wl["name"]
    t_setup = time.perf_counter()
    if workload == 3:
        step_layers = [B.stack()]
        replicas = 1
    else:
        touched = expert_bytes_per_expert(H, I, fmt) * min(E, T * K)
        replicas = B.args.replicas or max(2, min(16, math.ceil(1.5 * 2 ** 30 / touched) + 1))
        step_layers = [[r] for r in B.single_layer(wl["zipf"], replicas)]
    x = B.Wl.to_device_bf16(S.activations(workload, T, outliers=wl["outliers"]))
    buf = moe.MoeBuffers(T, H, I, E, K)
    n_layers = len(step_layers[0])
    if chain:
        norms = [moe.BranchNorms(*[B.Wl.to_device_bf16(a) for a in S.norm_weights(l)])
                 for l in range(n_layers)]
        xs = [x] + [torch.empty_like(x) for _ in range(n_layers)]
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    hs, stream = B.hs, B.stream
    separate = B.args.separate_prep
    # decode batches run as moe_layer_decode (three or four launches) unless a
    # variant asks for the separate calls
    fused = buf.decode and not (chain or separate or B.args.four_calls)
    stage_names = ("layer_decode",) if fused else SEPARATE_STAGES if separate else STAGES

    def stage_calls(layer, li):
        """The stage calls of one block pass (layer li of the step), by name."""
        x_in = xs[li] if chain else x
        nm = norms[li] if chain else None
        if chain:
            prep = lambda: C.nvfp4_expert_prep_rmsnorm(x_in, nm.pre2, nm.eps, E, I, K, buf.ws,
                                                       stream)
            combine = lambda: C.moe_combine_rmsnorm(buf.y_sorted, buf.topk_w, buf.pair_rank,
                                                    nm.post2, nm.eps, xs[li + 1],
                                                    post_norm=nm.post, residual=x_in,
                                                    layer_scalar=nm.layer_scalar, stream=stream)
        else:
            prep = lambda: C.nvfp4_expert_prep(x_in, E, I, K, buf.ws, stream)
            combine = lambda: C.moe_combine(buf.y_sorted, buf.topk_w, buf.pair_rank, buf.out,
                                            stream)
        return {
            "route_bucket_prep": lambda: C.moe_route_bucket_prep(
                x_in, layer.w_router, layer.router_scale, layer.per_expert_scale,
                layer.logit_bias, K, layer.eps, buf.topk_idx, buf.topk_w, buf.topk_w_raw,
                buf.logits, buf.expert_offsets, buf.sorted_pairs, buf.pair_rank, buf.bucket_ws,
                nm.pre2 if chain else None, nm.eps if chain else 0.0, I, buf.ws, stream),
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
            "layer_decode": lambda: C.moe_layer_decode(
                x_in, layer.w_router, layer.router_scale, layer.per_expert_scale,
                layer.logit_bias, K, layer.eps, layer.gate, layer.up, layer.down, buf.topk_idx,
                buf.topk_w, buf.topk_w_raw, buf.expert_offsets, buf.sorted_pairs, buf.pair_rank,
                buf.out, buf.layer_ws, stream),
        }

    def queue_step(layers):
        for li, layer in enumerate(layers):
            c = stage_calls(layer, li)
            if fused:
                c["layer_decode"]()
                continue
            if separate:
                c["prep"]()
                c["route_bucket"]()
            else:
                c["route_bucket_prep"]()
            c["gate_up"]()
            c["down"]()
            c["combine"]()

    for s in range(warmup):
        queue_step(step_layers[s % len(step_layers)])
    torch.cuda.synchronize()
    plan = [step_layers[(warmup + s) % len(step_layers)] for s in range(steps)]

    # ---- timed region: the K steps as one graph, replayed once
    graph = hip.instantiate(hip.capture(hs, lambda: [queue_step(p) for p in plan]))
    hip.launch(graph, hs)                       # one untimed replay
    torch.cuda.synchronize()
    gpu_ms, wall_ms, cold_ms = hip.timed_replay(graph, hs, torch.cuda.synchronize)
    ms_per_step = gpu_ms / steps

    # ---- the dominant kernel alone: the gate/up stage call R times back to
    # back (the same routing and buffers, the layers of the step plan in
    # turn, so the weights stream from HBM as in the steps) between two
    # events on the launch stream; the event cost spreads over R
    # (the decode path's gate/up kernel has no call of its own: its duration
    # comes from the kernel trace)
    gu_us, gu_graph = None, None
    if not fused:
        gu_calls = [stage_calls(layers[li], li)["gate_up"] for layers in plan
                    for li in range(len(layers))]
        reps_gu = max(20, len(gu_calls))
        gu_seq = [gu_calls[i % len(gu_calls)] for i in range(reps_gu)]
        gu_graph = hip.instantiate(hip.capture(hs, lambda: [c() for c in gu_seq]))
        hip.launch(gu_graph, hs)                # warm
        gu_ms, _, _ = hip.timed_replay(gu_graph, hs, torch.cuda.synchronize)
        gu_us = 1e3 * gu_ms / reps_gu

    stage_avg_us = None
    if stages:
        calls = []
        for layers in plan:
            for li, layer in enumerate(layers):
                c = stage_calls(layer, li)
                calls += [c[n] for n in stage_names]
        bounds = [hip.event() for _ in range(len(calls) + 1)]
        tg = hip.timed_chain(hs, calls, bounds)
        hip.launch(tg, hs)
        torch.cuda.synchronize()
        ms = {n: [] for n in stage_names}
        for j in range(len(calls)):
            ms[stage_names[j % len(stage_names)]].append(hip.elapsed(bounds[j], bounds[j + 1]))
        stage_avg_us = {n: 1e3 * float(np.mean(v)) for n, v in ms.items()}
        hip.h.hipGraphExecDestroy(tg)

    # ---- work done per step (realised routing)
    counts = np.diff(buf.expert_offsets.cpu().numpy())
    U_last = int((counts > 0).sum())            # the routing the gate/up launches ran on
    if n_layers > 1:
        U_total = 0
        for li, layer in enumerate(step_layers[0]):
            stage_calls(layer, li)["layer_decode" if fused else "route_bucket_prep"]()
            torch.cuda.synchronize()
            U_total += int((np.diff(buf.expert_offsets.cpu().numpy()) > 0).sum())
    else:
        U_total = U_last
    P = T * K
    per_exp = expert_bytes_per_expert(H, I, fmt)
    gu_w_bytes = 2 * proj_bytes(H, I, fmt)
    step_s = ms_per_step / 1e3
    gate_up_alg_bytes = gu_w_bytes * U_last + T * H * 2 + P * I * 2     # per launch
    gu_flops = 2.0 * P * 2 * I * H
    gu_gbps = gate_up_alg_bytes / (gu_us * 1e-6) / 1e9 if gu_us else None
    gu_tflops = gu_flops / (gu_us * 1e-6) / 1e12 if gu_us else None
    expert_flops = 2.0 * P * 3 * I * H * n_layers
    prefill = workload in (2, 4)
    res = {
        "workload": name, "tokens": T, "layers": n_layers, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "ms_per_step_wall": wall_ms / steps,
        "ms_per_step_launch_on_idle_stream": cold_ms / steps,
        "tokens_per_s": T / step_s,
        "active_experts": U_total,
        "expert_weight_GBps": per_exp * U_total / step_s / 1e9,
        "layer_alg_GBps": (per_exp * U_total + n_layers * ((E * H + H + E) * 2 + 2 * T * H * 2))
                          / step_s / 1e9,
        "expert_TFLOPs": expert_flops / step_s / 1e12,
        "max_over_mean_bucket": float(counts.max() / max(counts.mean(), 1e-9)),
        "weight_replicas": replicas, "setup_s": t_setup,
        "gate_up_kernel": ("k_decode_gate_up (in moe_layer_decode)" if fused else
                           gate_up_kernel_name(T, K, E, fmt)), "gate_up_us": gu_us,
        "gate_up_GBps": gu_gbps, "gate_up_TFLOPs": gu_tflops,
        "gate_up_frac": (None if not gu_us else gu_tflops / F16_MFMA_PEAK_TFLOPS if prefill
                         else gu_gbps / HBM_PEAK_GBPS),
        "gate_up_bound": "mfma" if prefill else "hbm",
        "_gate_up_alg_bytes": gate_up_alg_bytes, "_gate_up_flops": gu_flops,
        "_U_last": U_last,
    }
    if stage_avg_us is not None:
        res["stage_avg_us_with_event_nodes"] = stage_avg_us
    res["path"] = ((f"moe_layer_decode ({3 if T * K <= 32 else 4} launches)") if fused else
                   "moe_route_bucket + nvfp4_expert_prep + gate_up + down + combine" if separate else
                   "moe_route_bucket_prep + nvfp4_expert_gate_up + nvfp4_expert_down + combine")
    for g in (graph, gu_graph):
        if g is not None:
            hip.h.hipGraphExecDestroy(g)
    return res


def roofline(res, workload):
    """The dominant kernel's roofline: the HBM one for decode (its algorithmic
    bytes: the active experts' gate and up tensors, the f16 activations and
    A written), the f16 MFMA one for prefill (its algorithmic flops
    2 P 2 I H); the other one beside it."""
    T, K, I, H = res["tokens"], 8, 704, 2816
    traffic = profiled_traffic(res["workload"], res["gate_up_kernel"])
    U, P = res["_U_last"], T * K
    w_bytes = res["_gate_up_alg_bytes"] - T * H * 2 - P * I * 2
    frac = lambda v, p: None if v is None else v / p
    hbm = {"kernel": res["gate_up_kernel"], "bound": "hbm", "achieved": res["gate_up_GBps"],
           "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": frac(res["gate_up_GBps"], HBM_PEAK_GBPS),
           "traffic": traffic, "alg_bytes_per_launch": res["_gate_up_alg_bytes"],
           "avg_launch_us": res["gate_up_us"],
           "units": f"{U} active experts x {w_bytes // max(U, 1)} B + {T} x {H} x 2 B + "
                    f"{P} x {I} x 2 B"}
    mfma = {"kernel": res["gate_up_kernel"], "bound": "mfma", "achieved": res["gate_up_TFLOPs"],
            "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": frac(res["gate_up_TFLOPs"], F16_MFMA_PEAK_TFLOPS), "traffic": traffic,
            "alg_flops_per_launch": res["_gate_up_flops"], "avg_launch_us": res["gate_up_us"],
            "units": f"2 x {P} rows x 2 x {I} x {H}"}
    return (mfma, hbm) if workload in (2, 4) else (hbm, mfma)


DTYPES = {"nvfp4": "nvfp4 weights (e2m1 x e4m3 x fp32) x bf16 activations; f16 MFMA, fp32 accumulate",
          "q4_0": "int4 q4_0 weights ((q - 8) x fp16 d per 32) x bf16 activations; f16 MFMA",
          "aff4": "int4 affine weights (q x fp16 s + fp16 b per 32) x bf16 activations; f16 MFMA"}
DATA = {"nvfp4": "synthetic (seeded; bf16 N(0,0.02) experts quantised to NVFP4 on the GPU)",
        "q4_0": "synthetic (seeded; uniform int4 codes, fp16 d ~ U(0.004, 0.008))",
        "aff4": "synthetic (seeded; uniform int4 codes, fp16 s ~ U(0.004, 0.008), "
                "b ~ U(-0.06, -0.035))"}


def public(res):
    return {k: v for k, v in res.items() if not k.startswith("_")}


def main(argv=None):
    args = parse(argv)
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

    torch.cuda.set_device(0)
    moe.lib()
    B = Bench(args)
    suffix = "" if args.format == "nvfp4" else f"_{args.format}"
    if args.workload is None:
        runs = list(ALL_RUNS)
    elif args.workload == 3:
        runs = [(3, args.sweep_T)]
    else:
        runs = [(args.workload, args.tokens or S.WORKLOADS[args.workload]["T"][0])]
    results = []
    for workload, T in runs:
        steps, warmup = step_defaults(workload, args.steps, args.warmup)
        name = S.WORKLOADS[workload]["name"]
        if workload == 3:
            name = f"moe_30layer_decode_sweep_T{T}" + ("_chained" if args.chain else "")
        elif T != S.WORKLOADS[workload]["T"][0]:
            name = re.sub(r"_T\d+", f"_T{T}", name)
        res = run_workload(B, workload, T, steps, warmup, stages=args.stages and not results,
                           chain=args.chain and workload == 3, name=name + suffix)
        results.append((workload, res))
        gu = ("" if res["gate_up_us"] is None else
              f", gate/up {res['gate_up_us']:.1f} us frac {res['gate_up_frac']:.3f}")
        print(f"# {res['workload']}: {res['ms_per_step'] * 1e3:.1f} us/step "
              f"({res['tokens_per_s']:.0f} tok/s, {res['path']}){gu}", file=sys.stderr,
              flush=True)
    head_w, head = results[0]
    rl, rl_other = roofline(head, head_w)
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s" if head_w != 3 else "tokens/s (30-layer sweep)",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[args.format],
        "data": DATA[args.format],
        "config": {"workload": head["workload"], "tokens": head["tokens"], "hidden": B.H,
                   "experts": B.E, "top_k": B.K, "moe_intermediate": B.I,
                   "layers": head["layers"], "weight_replicas": head["weight_replicas"],
                   "timing": "hip_graph (one stream); GPU time by HIP events around the second of two back-to-back replays"},
        "detail": {"headline": public(head),
                   "workloads": {r["workload"]: public(r) for _, r in results[1:]}},
        "roofline": rl,
        ("roofline_hbm" if rl["bound"] == "mfma" else "roofline_mfma"): rl_other,
    }
    if not args.no_cpu_baseline and head_w != 3:
        out["cpu_baseline"] = cpu_baseline(args, S.WORKLOADS[head_w], head_w, head["tokens"])
    print(json.dumps(out), flush=True)


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


def cpu_baseline(args, wl, workload, T):
    """The fp64 oracle as it stands on a bounded sample of the same workload:
    the block for the first n tokens (expert weights quantised by the oracle
    itself beforehand, untimed), its BLAS calls on every core of the
    process's affinity set."""
    from threadpoolctl import threadpool_limits
    import moe_synth as S
    from oracle import formats as F
    from oracle import int4 as Q
    from oracle import moe as M
    from oracle.quantize import quantize
    from concurrent.futures import ThreadPoolExecutor

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    n = min(T, args.cpu_sample_tokens)
    p = S.router_params(0, zipf=wl["zipf"])
    r = dict(w_router=F.bf16_bits_to_f64(p["w_router"]), scale=F.bf16_bits_to_f64(p["scale"]),
             per_expert_scale=F.bf16_bits_to_f64(p["per_expert_scale"]), bias=p["bias"])
    x = F.bf16_bits_to_f64(S.activations(workload, T, outliers=wl["outliers"]))[:n]
    ids = M.route(x, r["w_router"], r["scale"], r["per_expert_scale"], 8, r["bias"])["idx"]
    todo = [(proj, int(e)) for e in np.unique(ids) for proj in (S.GATE, S.UP, S.DOWN)]
    fmt = args.format

    def q(item):
        proj, e = item
        if fmt != "nvfp4":
            return item, S.int4_expert(fmt, 0, proj, e)
        return item, quantize(F.bf16_bits_to_f64(S.expert_weight(0, proj, e)))

    with ThreadPoolExecutor(cores) as ex:
        packed = dict(ex.map(q, todo))                    # weight preparation, untimed

    def decode(item):
        if fmt == "nvfp4":
            return F.dequantize(*packed[item])
        pk, sb = packed[item]
        bits = sb.view(np.uint16)
        if fmt == "q4_0":
            return Q.decode_q4_0(pk, bits)
        return Q.decode_aff4(pk, bits.reshape(bits.shape[0], -1, 2))
    fn = {proj: (lambda e, proj=proj: decode((proj, e))) for proj in (S.GATE, S.UP, S.DOWN)}
    # the same block again until at least 10 s have been timed (the expert
    # decode, not the token count, dominates one run)
    runs, dt = 0, 0.0
    with threadpool_limits(cores):
        while runs == 0 or (dt < 10.0 and runs < 8):
            t0 = time.perf_counter()
            M.moe_block(x, x, r, fn[S.GATE], fn[S.UP], fn[S.DOWN], k=8)
            dt += time.perf_counter() - t0
            runs += 1
    return {"value": n * runs / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of the {T} tokens of {wl['name']} through the fp64 oracle block "
                      f"(route, bucket, {fmt} decode of the {len(todo) // 3} touched experts, "
                      f"expert MLPs, combine), {runs} run(s) in {dt:.1f} s; BLAS on {cores} "
                      f"threads, the numpy expert decode single-threaded"}


if __name__ == "__main__":
    main()
