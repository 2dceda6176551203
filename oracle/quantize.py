"""NVFP4 block quantiser in float64 (oracle; test infrastructure only).

"Gemma-4-26B-A4B-it-NVFP4" README, block-quantisation formulas: weights are cut
into contiguous blocks of 16 along the inner (input) dimension; each block gets
S_block = max_i |w_i| / V_max with V_max = 6, the largest E2M1 magnitude; each
weight becomes q_i = clip(round(w_i / S_block), -V_max, V_max) and is
reconstructed as ŵ_i = q_i * S_block.  "Two-level" (the NVFP4-mlx Quantization
recipe table) splits S_block into an E4M3 block scale times one FP32 scale per
tensor.

Readings (the pages leave these open):
* The per-tensor FP32 scale is g = fl32(max|W| / (6 * 448)), so that the
  largest block scale lands on the largest E4M3 value; one g per (expert,
  projection) tensor.
* The E4M3 block scale code is the nearest E4M3 value (ties to even, saturating
  at 448) to amax_block / (6 g); the block's effective scale is E4M3(code) * g.
* "round" in q_i means: nearest E2M1 value, ties to the even code, after the
  clip to [-6, 6].  A block whose scale is 0 gets all-zero codes.
* Everything is evaluated in float64 from the bf16 input values; fp64 division
  is correctly rounded, so a port evaluating the same expressions in IEEE
  double reaches the same codes.
"""
import numpy as np

from .formats import (E2M1_MAX, E4M3_MAX, e2m1_encode, e4m3_decode, e4m3_encode,
                      pack_nibbles)

GROUP = 16


def global_scale(w):
    """g = fl32(max|W| / (6 * 448)) as a float64 holding an fp32 value."""
    amax = float(np.max(np.abs(w))) if w.size else 0.0
    return float(np.float32(amax / (E2M1_MAX * E4M3_MAX)))


def quantize(w, group=GROUP):
    """Quantise one tensor w [N, K] (float64 of bf16 values), K % 16 == 0.

    Returns (packed uint8 [N, K/2], scale codes uint8 [N, K/16], g float).
    """
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    g = global_scale(w)
    blocks = w.reshape(n, k // group, group)
    if g == 0.0:
        return (np.zeros((n, k // 2), np.uint8), np.zeros((n, k // group), np.uint8), 0.0)
    amax_b = np.abs(blocks).max(axis=-1)
    r_b = amax_b / (E2M1_MAX * g)
    sc = e4m3_encode(r_b)
    s_b = e4m3_decode(sc) * g                      # exact in float64
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s_b[..., None] > 0, blocks / s_b[..., None], 0.0)
    ratio = np.clip(ratio, -E2M1_MAX, E2M1_MAX)
    codes = e2m1_encode(ratio).reshape(n, k)
    return pack_nibbles(codes), sc.astype(np.uint8), g


def quantize_experts(w_stack, group=GROUP):
    """Per-expert quantisation of a stack [E, N, K]: one g per expert."""
    outs = [quantize(w_stack[e], group) for e in range(w_stack.shape[0])]
    packed = np.stack([o[0] for o in outs])
    scales = np.stack([o[1] for o in outs])
    gs = np.array([o[2] for o in outs], dtype=np.float64)
    return packed, scales, gs
