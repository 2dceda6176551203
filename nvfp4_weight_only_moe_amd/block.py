"""One MoE expert block as the sequence of the four C-ABI calls.

``MoeLayer`` holds one layer's device weights, ``MoeBuffers`` the caller-owned
outputs and workspaces for a token count, ``forward`` queues the block on one
stream: moe_route_bucket_prep (router, bucketing and the expert-input prep of
the same x) -> nvfp4_expert_gate_up -> nvfp4_expert_down -> moe_combine, the
same results as moe_route -> moe_bucket -> nvfp4_expert_mlp -> moe_combine.
Nothing here computes: it only allocates device memory and passes pointers.
"""
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib


@dataclass
class MoeLayer:
    w_router: torch.Tensor          # [E, H] bf16
    router_scale: torch.Tensor      # [H] bf16
    per_expert_scale: torch.Tensor  # [E] bf16
    logit_bias: Optional[torch.Tensor]  # [E] f32 or None
    gate: "_lib.Nvfp4Weights"       # [E, I, H]
    up: "_lib.Nvfp4Weights"         # [E, I, H]
    down: "_lib.Nvfp4Weights"       # [E, H, I]
    top_k: int = 8
    eps: float = 1e-6

    @property
    def E(self):
        return self.w_router.shape[0]

    @property
    def H(self):
        return self.w_router.shape[1]

    @property
    def I(self):
        return self.gate.N

    def with_experts(self, gate, up, down):
        return MoeLayer(self.w_router, self.router_scale, self.per_expert_scale, self.logit_bias,
                        gate, up, down, self.top_k, self.eps)


class MoeBuffers:
    """Every output and workspace of the four calls for T tokens."""

    def __init__(self, T, H, I, E, top_k, device="cuda"):
        kw = dict(device=device)
        P = T * top_k
        self.T, self.P = T, P
        self.logits = torch.empty((T, E), dtype=torch.float32, **kw)
        self.topk_idx = torch.empty((T, top_k), dtype=torch.int32, **kw)
        self.topk_w = torch.empty((T, top_k), dtype=torch.float32, **kw)
        self.topk_w_raw = torch.empty((T, top_k), dtype=torch.float32, **kw)
        self.expert_offsets = torch.empty((E + 1,), dtype=torch.int32, **kw)
        self.sorted_pairs = torch.empty((P,), dtype=torch.int32, **kw)
        self.pair_rank = torch.empty((P,), dtype=torch.int32, **kw)
        self.bucket_ws = torch.empty((_lib.moe_bucket_workspace_bytes(T, top_k, E),),
                                     dtype=torch.uint8, **kw)
        self.ws = torch.empty((_lib.moe_workspace_bytes(T, top_k, E, H, I),), dtype=torch.uint8, **kw)
        self.y_sorted = torch.empty((P, H), dtype=torch.bfloat16, **kw)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, **kw)
        # the three-launch decode path's workspace (small batches only)
        self.decode = _lib.decode_fits(T, top_k, H)
        self.layer_ws = None
        if self.decode:
            self.layer_ws = torch.empty((_lib.moe_layer_decode_workspace_bytes(T, top_k, E, H, I),),
                                        dtype=torch.uint8, **kw)
            self._decode_err = _lib.moe_layer_decode_error_offset(T, top_k, E)
        self._err_src = self.bucket_ws[:4]
        self.y_sorted_valid = False  # y_sorted holds the last four-call pass's expert outputs

    def bucket_error_count(self):
        """Pairs whose expert id was out of range in the last bucketing."""
        return int(self._err_src.view(torch.int32)[0].item())


def forward(layer: MoeLayer, x, buf: MoeBuffers, x_expert=None, stream=None, marks=None,
            fused=None):
    """Queue the whole block for x [T, H] bf16; the result lands in buf.out.

    Decode batches (T <= 8) run as moe_layer_decode (three or four launches) unless
    ``fused`` is False or the experts read another input.  ``marks``
    (optional) is a callable invoked with a stage name between the calls
    ("route", "bucket", "prep", "gate_up", "down", "combine" after each); with
    it the block runs as the separate stage calls so that a caller can record
    timing events around each stage."""
    xe = x if x_expert is None else x_expert
    mark = marks or (lambda name: None)
    if fused is None:
        fused = buf.decode and x_expert is None and marks is None
    if fused:
        _lib.moe_layer_decode(x, layer.w_router, layer.router_scale, layer.per_expert_scale,
                              layer.logit_bias, layer.top_k, layer.eps, layer.gate, layer.up,
                              layer.down, buf.topk_idx, buf.topk_w, buf.topk_w_raw,
                              buf.expert_offsets, buf.sorted_pairs, buf.pair_rank, buf.out,
                              buf.layer_ws, stream)
        buf._err_src = buf.layer_ws[buf._decode_err:buf._decode_err + 4]
        buf.y_sorted_valid = False   # the expert outputs are in the call's workspace
        return buf.out
    buf._err_src = buf.bucket_ws[:4]
    buf.y_sorted_valid = True
    if marks is None and x_expert is None:
        # the router and the expert-input prep read the same x: one call
        _lib.moe_route_bucket_prep(x, layer.w_router, layer.router_scale, layer.per_expert_scale,
                                   layer.logit_bias, layer.top_k, layer.eps, buf.topk_idx,
                                   buf.topk_w, buf.topk_w_raw, buf.logits, buf.expert_offsets,
                                   buf.sorted_pairs, buf.pair_rank, buf.bucket_ws, None, 0.0,
                                   layer.I, buf.ws, stream)
        _lib.nvfp4_expert_gate_up(layer.gate, layer.up, buf.expert_offsets, buf.sorted_pairs,
                                  buf.T, layer.top_k, layer.H, buf.ws, stream)
        _lib.nvfp4_expert_down(layer.down, buf.expert_offsets, buf.T, layer.top_k, buf.y_sorted,
                               buf.ws, stream)
        _lib.moe_combine(buf.y_sorted, buf.topk_w, buf.pair_rank, buf.out, stream)
        return buf.out
    if marks is None:
        _lib.moe_route_bucket(x, layer.w_router, layer.router_scale, layer.per_expert_scale,
                              layer.logit_bias, layer.top_k, layer.eps, buf.topk_idx, buf.topk_w,
                              buf.topk_w_raw, buf.logits, buf.expert_offsets, buf.sorted_pairs,
                              buf.pair_rank, buf.bucket_ws, stream)
    else:
        _lib.moe_route(x, layer.w_router, layer.router_scale, layer.per_expert_scale,
                       layer.logit_bias, layer.top_k, layer.eps, buf.topk_idx, buf.topk_w,
                       buf.topk_w_raw, buf.logits, stream)
        mark("route")
        _lib.moe_bucket(buf.topk_idx, layer.E, buf.expert_offsets, buf.sorted_pairs,
                        buf.pair_rank, buf.bucket_ws, stream)
        mark("bucket")
    if marks is None:
        _lib.nvfp4_expert_mlp(xe, layer.gate, layer.up, layer.down, buf.expert_offsets,
                              buf.sorted_pairs, layer.top_k, buf.y_sorted, buf.ws, stream)
    else:
        _lib.nvfp4_expert_prep(xe, layer.E, layer.I, layer.top_k, buf.ws, stream)
        mark("prep")
        _lib.nvfp4_expert_gate_up(layer.gate, layer.up, buf.expert_offsets, buf.sorted_pairs,
                                  buf.T, layer.top_k, layer.H, buf.ws, stream)
        mark("gate_up")
        _lib.nvfp4_expert_down(layer.down, buf.expert_offsets, buf.T, layer.top_k, buf.y_sorted,
                               buf.ws, stream)
        mark("down")
    _lib.moe_combine(buf.y_sorted, buf.topk_w, buf.pair_rank, buf.out, stream)
    mark("combine")
    return buf.out


@dataclass
class BranchNorms:
    """The learned norms of the layer step around the sparse branch ("Gemma 4
    26B-A4B (MoE) - Core AI", Architecture sketch) and its layer scalar."""
    pre2: torch.Tensor                    # [H] bf16, pre_feedforward_layernorm_2
    post2: torch.Tensor                   # [H] bf16, post_feedforward_layernorm_2
    post: Optional[torch.Tensor] = None   # [H] bf16, post_feedforward_layernorm (None: h2 only)
    eps: float = 1e-6
    layer_scalar: float = 1.0


def forward_branch(layer: MoeLayer, residual, buf: MoeBuffers, norms: BranchNorms, h1=None,
                   stream=None):
    """The sparse branch with its norms and the layer step: the router reads
    the raw residual, the experts read rmsnorm(residual, pre2), h2 =
    rmsnorm(sum_k w_k y_k, post2), and buf.out = (residual + rmsnorm(h1 + h2,
    post)) * layer_scalar (h1: the dense branch's output, None for zero).
    Without ``norms.post`` buf.out is h2."""
    _lib.moe_route_bucket_prep(residual, layer.w_router, layer.router_scale,
                               layer.per_expert_scale, layer.logit_bias, layer.top_k, layer.eps,
                               buf.topk_idx, buf.topk_w, buf.topk_w_raw, buf.logits,
                               buf.expert_offsets, buf.sorted_pairs, buf.pair_rank, buf.bucket_ws,
                               norms.pre2, norms.eps, layer.I, buf.ws, stream)
    _lib.nvfp4_expert_gate_up(layer.gate, layer.up, buf.expert_offsets, buf.sorted_pairs, buf.T,
                              layer.top_k, layer.H, buf.ws, stream)
    _lib.nvfp4_expert_down(layer.down, buf.expert_offsets, buf.T, layer.top_k, buf.y_sorted,
                           buf.ws, stream)
    buf._err_src = buf.bucket_ws[:4]
    buf.y_sorted_valid = True
    step = norms.post is not None
    _lib.moe_combine_rmsnorm(buf.y_sorted, buf.topk_w, buf.pair_rank, norms.post2, norms.eps,
                             buf.out, h1=h1 if step else None, post_norm=norms.post,
                             residual=residual if step else None,
                             layer_scalar=norms.layer_scalar, stream=stream)
