"""Device-resident synthetic workloads: seeded bf16 inputs from ``moe_synth``,
uploaded once, expert weights quantised on the GPU by ``nvfp4_quantize`` (or,
for the int4 formats, uploaded as drawn and repacked)."""
import numpy as np
import torch

import moe_synth as S

from . import _lib
from .block import MoeLayer


def to_device_bf16(bits, device="cuda"):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on the device."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def quantize_stack_on_gpu(bits_stack, device="cuda", chunk=32, tiled=True):
    """[E, N, K] bf16 bits -> Nvfp4Weights, uploaded and quantised in chunks,
    then (by default) repacked into the tiled layout the expert kernels read."""
    E, N, K = bits_stack.shape
    out = _lib.Nvfp4Weights.empty(E, N, K, device)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        w = to_device_bf16(bits_stack[e0:e1], device)
        _lib.nvfp4_quantize(w, out.select(e0, e1))
    return _lib.nvfp4_repack(out) if tiled else out


def router_to_device(p, device="cuda"):
    bias = None if p["bias"] is None else torch.from_numpy(p["bias"]).to(device)
    return (to_device_bf16(p["w_router"], device), to_device_bf16(p["scale"], device),
            to_device_bf16(p["per_expert_scale"], device), bias)


def build_layer(layer=0, zipf=False, device="cuda", seed=S.SEED, h=S.H, i=S.I, e=S.E, k=S.TOP_K,
                experts_chunk=32):
    """One layer of the model-shaped workload on the device."""
    wr, sc, pes, bias = router_to_device(S.router_params(layer, seed, h, e, zipf), device)
    stacks = []
    for proj in (S.GATE, S.UP, S.DOWN):
        n, kk = S.proj_shape(proj, h, i)
        out = _lib.Nvfp4Weights.empty(e, n, kk, device)
        buf = np.empty((experts_chunk, n, kk), dtype=np.uint16)
        for e0 in range(0, e, experts_chunk):
            e1 = min(e, e0 + experts_chunk)
            S.expert_weights(layer, proj, range(e0, e1), seed, h, i, out=buf[:e1 - e0])
            _lib.nvfp4_quantize(to_device_bf16(buf[:e1 - e0], device), out.select(e0, e1))
        stacks.append(_lib.nvfp4_repack(out))
        del out
    torch.cuda.synchronize()
    return MoeLayer(wr, sc, pes, bias, stacks[0], stacks[1], stacks[2], k)


def build_small_layer(case, top_k, device="cuda"):
    """A ``moe_synth.small_case`` dict on the device (weights quantised on GPU)."""
    r = case["router"]
    wr, sc, pes, bias = router_to_device(r, device)
    g = quantize_stack_on_gpu(case["gate"], device)
    u = quantize_stack_on_gpu(case["up"], device)
    d = quantize_stack_on_gpu(case["down"], device)
    return MoeLayer(wr, sc, pes, bias, g, u, d, top_k=top_k)


def int4_to_device(fmt, packed, scales, device="cuda", tiled=True):
    """An int4 stack (``moe_synth`` arrays: packed [E, N, K/2] u8, scale bytes
    [E, N, ...] u8) as Nvfp4Weights of format ``fmt`` ("q4_0" or "aff4")."""
    w = _lib.Nvfp4Weights(torch.from_numpy(np.ascontiguousarray(packed)).to(device),
                          torch.from_numpy(np.ascontiguousarray(scales)).to(device), None,
                          _lib.LAYOUT_CANONICAL, _lib.FORMATS[fmt])
    return _lib.nvfp4_repack(w) if tiled else w


def build_int4_layer(fmt, layer=0, zipf=False, device="cuda", seed=S.SEED, h=S.H, i=S.I, e=S.E,
                     k=S.TOP_K):
    """One model-shaped layer with int4 expert stacks of format ``fmt``."""
    wr, sc, pes, bias = router_to_device(S.router_params(layer, seed, h, e, zipf), device)
    stacks = [int4_to_device(fmt, *S.int4_stack(fmt, layer, proj, seed, h, i, e), device=device)
              for proj in (S.GATE, S.UP, S.DOWN)]
    torch.cuda.synchronize()
    return MoeLayer(wr, sc, pes, bias, stacks[0], stacks[1], stacks[2], k)


def build_small_int4_layer(case, fmt, top_k, device="cuda"):
    """A ``moe_synth.small_int4_case`` dict on the device."""
    wr, sc, pes, bias = router_to_device(case["router"], device)
    g, u, d = (int4_to_device(fmt, *case[n], device=device) for n in ("gate", "up", "down"))
    return MoeLayer(wr, sc, pes, bias, g, u, d, top_k=top_k)


def replicate_experts(layer, n, device="cuda"):
    """n byte-identical copies of a layer's expert weights (distinct memory),
    used to time HBM streaming rather than cache hits."""
    reps = [layer]
    for _ in range(n - 1):
        cp = [w.clone() for w in (layer.gate, layer.up, layer.down)]
        reps.append(layer.with_experts(*cp))
    return reps
