"""NVFP4 expert stacks from the two-level checkpoint layout.

"Gemma-4-26B-A4B-NVFP4-mlx" (opening paragraph and Quantization recipe): the
published checkpoint ships each expert projection as packed-U8 NVFP4 codes with
a ``weight_scale`` sidecar (one E4M3 code per 16 weights along K) and a
``weight_scale_2`` sidecar (the per-tensor FP32 scale).  The same page ("How it
was made") stacks the experts as ``gate_up_proj [128, 1408, 2816]`` with gate
and up fused, and ``down_proj [128, 2816, 704]``.

This module turns such tensors into the library's stacks: it splits the fused
gate/up stack (gate rows first), brings the scales to one FP32 value per
expert, and repacks on the device into the tiled layout the expert kernels
read.  It is weight preparation, run once; nothing here is on the hot path.

Readings of the layout (the pages name the sidecars but not their encoding):
* ``packed [E, N, K/2]`` u8, the code of the even k in the low nibble;
* ``weight_scale [E, N, K/16]`` E4M3 codes (u8, or torch.float8_e4m3fn viewed
  as bytes);
* ``weight_scale_2`` multiplies (w = E2M1 x E4M3 x scale_2); one value for
  the whole stack, or one per expert ([E], [E, 1] or [E, 1, 1]).  A checkpoint
  that stores the reciprocal passes 1 / value;
* a fused stack of 2*I rows holds gate in rows [0, I) and up in [I, 2*I).
"""
import torch

from . import _lib


def _u8(t, name):
    if t.dtype == torch.uint8:
        return t
    if t.element_size() == 1:
        return t.view(torch.uint8)
    raise TypeError(f"{name}: expected 1-byte elements, got {t.dtype}")


def stack_from_two_level(packed, weight_scale, weight_scale_2, device="cuda"):
    """One canonical NVFP4 stack from the checkpoint's tensors (copied to
    ``device``)."""
    packed = _u8(packed, "packed")
    scales = _u8(weight_scale, "weight_scale")
    if packed.dim() != 3 or scales.dim() != 3:
        raise ValueError("packed and weight_scale must be [E, N, K/2] and [E, N, K/16]")
    E, N, k2 = packed.shape
    if tuple(scales.shape) != (E, N, 2 * k2 // 16) or (2 * k2) % 16:
        raise ValueError(f"weight_scale shape {tuple(scales.shape)} does not match packed "
                         f"{tuple(packed.shape)}")
    g = torch.as_tensor(weight_scale_2, dtype=torch.float32).reshape(-1)
    if g.numel() == 1:
        g = g.expand(E)
    elif g.numel() != E:
        raise ValueError(f"weight_scale_2 has {g.numel()} values for {E} experts")
    return _lib.Nvfp4Weights(packed.to(device).contiguous(), scales.to(device).contiguous(),
                             g.to(device).contiguous().clone(), _lib.LAYOUT_CANONICAL)


def split_gate_up(fused):
    """(gate, up) canonical stacks from a fused [E, 2*I, K] stack (copies)."""
    if fused.layout != _lib.LAYOUT_CANONICAL:
        raise ValueError("split_gate_up takes the canonical layout")
    if fused.N % 2:
        raise ValueError("a fused gate/up stack has an even row count")
    i = fused.N // 2

    def rows(a, b):
        return _lib.Nvfp4Weights(fused.packed[:, a:b].contiguous(),
                                 fused.scales[:, a:b].contiguous(), fused.global_scale.clone(),
                                 _lib.LAYOUT_CANONICAL)
    return rows(0, i), rows(i, 2 * i)


def load_experts(gate_up, down, device="cuda", tiled=True, stream=None):
    """gate_up, down: (packed, weight_scale, weight_scale_2) of the fused
    gate/up stack and of the down stack.  Returns (gate, up, down) stacks,
    repacked on the device into the tiled layout unless ``tiled`` is false."""
    gate, up = split_gate_up(stack_from_two_level(*gate_up, device=device))
    dn = stack_from_two_level(*down, device=device)
    if gate.K != dn.N or dn.K != gate.N:
        raise ValueError(f"gate/up [{gate.N}, {gate.K}] and down [{dn.N}, {dn.K}] do not chain")
    if not tiled:
        return gate, up, dn
    return tuple(_lib.nvfp4_repack(w, stream) for w in (gate, up, dn))


def load_experts_safetensors(path, gate_up_name, down_name, device="cuda", tiled=True,
                             scale_suffix=".weight_scale", scale2_suffix=".weight_scale_2"):
    """load_experts from a safetensors file: the packed codes under
    ``gate_up_name`` / ``down_name`` and the sidecars under the same names
    plus the suffixes."""
    from safetensors.torch import load_file
    t = load_file(path)

    def triple(name):
        return t[name], t[name + scale_suffix], t[name + scale2_suffix]
    return load_experts(triple(gate_up_name), triple(down_name), device, tiled)
