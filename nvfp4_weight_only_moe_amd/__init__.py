"""NVFP4 weight-only Gemma-4-26B-A4B MoE expert block for MI355X (gfx950).

The product is the HIP library ``libmoe_nvfp4.so`` behind the C ABI in
``include/moe_nvfp4.h``; this package is its thin Python binding (``_lib``),
the four-call block sequence (``block``), device-resident synthetic
workloads (``workload``) and the loader of two-level NVFP4 checkpoint tensors
(``checkpoint``).
"""
from ._lib import (EXPORTED, FORMAT_AFF4, FORMAT_NVFP4, FORMAT_Q4_0, FORMATS, LAYOUT_CANONICAL,
                   LAYOUT_TILED, MoeError, Nvfp4Weights, lib, moe_bucket,
                   moe_bucket_workspace_bytes, moe_combine, moe_combine_rmsnorm,
                   moe_dequant_f16, moe_route, moe_route_bucket, moe_route_bucket_prep,
                   moe_workspace_bytes, nvfp4_dequant_bf16, nvfp4_expert_down, nvfp4_expert_gate_up,
                   nvfp4_expert_mlp, nvfp4_expert_mlp_noalloc, nvfp4_expert_prep, nvfp4_expert_prep_rmsnorm, nvfp4_quantize,
                   nvfp4_repack)
from .block import BranchNorms, MoeBuffers, MoeLayer, forward, forward_branch

__all__ = ["EXPORTED", "MoeError", "Nvfp4Weights", "lib", "moe_bucket", "moe_bucket_workspace_bytes",
           "moe_combine", "moe_combine_rmsnorm", "nvfp4_expert_prep_rmsnorm", "moe_route", "moe_route_bucket", "moe_route_bucket_prep", "moe_workspace_bytes", "nvfp4_dequant_bf16",
           "nvfp4_expert_mlp", "nvfp4_expert_mlp_noalloc", "nvfp4_expert_prep", "nvfp4_expert_gate_up", "nvfp4_expert_down",
           "nvfp4_quantize", "nvfp4_repack", "LAYOUT_CANONICAL", "LAYOUT_TILED", "MoeBuffers",
           "MoeLayer", "forward", "BranchNorms", "forward_branch", "moe_dequant_f16",
           "FORMAT_NVFP4", "FORMAT_Q4_0", "FORMAT_AFF4", "FORMATS"]
