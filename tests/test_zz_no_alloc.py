"""The allocation-free expert MLP entry point (nvfp4_expert_mlp_noalloc, the
library's own per-GPU scratch array instead of a caller workspace) against
nvfp4_expert_mlp with a caller workspace: the same output bytes, on two calls
in a row, the second with a smaller input."""
import ctypes

import numpy as np
import pytest
import torch

import moe_synth as S
import nvfp4_weight_only_moe_amd as moe
from nvfp4_weight_only_moe_amd import _lib
from nvfp4_weight_only_moe_amd import workload as W

pytestmark = pytest.mark.gpu


def _route(layer, T, seed):
    x = W.to_device_bf16(S.activations(seed, T, h=layer.H))
    buf = moe.MoeBuffers(T, layer.H, layer.I, layer.E, layer.top_k)
    moe.moe_route_bucket(x, layer.w_router, layer.router_scale, layer.per_expert_scale,
                         layer.logit_bias, layer.top_k, layer.eps, buf.topk_idx, buf.topk_w,
                         buf.topk_w_raw, buf.logits, buf.expert_offsets, buf.sorted_pairs,
                         buf.pair_rank, buf.bucket_ws)
    return x, buf


def _both(layer, T, seed):
    x, buf = _route(layer, T, seed)
    k = layer.top_k
    ref = torch.empty((T * k, layer.H), dtype=torch.bfloat16, device="cuda")
    moe.nvfp4_expert_mlp(x, layer.gate, layer.up, layer.down, buf.expert_offsets,
                         buf.sorted_pairs, k, ref, buf.ws)
    got = torch.full((T * k, layer.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.nvfp4_expert_mlp_noalloc(x, layer.gate, layer.up, layer.down, buf.expert_offsets,
                                 buf.sorted_pairs, k, got)
    torch.cuda.synchronize()
    return got, ref


@pytest.fixture(scope="module")
def model_layer():
    assert torch.cuda.is_available()
    moe.lib()
    return W.build_layer(0)


def test_noalloc_matches_workspace_call_model_shape(model_layer):
    # decode batch (GEMV mode), then a smaller one on the same scratch array
    for T, seed in ((64, 71), (5, 72)):
        got, ref = _both(model_layer, T, seed)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), T


def test_noalloc_matches_workspace_call_gemm_mode():
    # a small block in the tiled GEMM mode (many rows per expert), then a
    # smaller GEMV-mode call after it
    k, E, H, I = 4, 16, 256, 128
    for T, seed in ((300, 81), (7, 82)):
        c = S.small_case(seed, T, H, I, E, k)
        layer = W.build_small_layer(c, k)
        got, ref = _both(layer, T, seed)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), T


def test_noalloc_rejects_sizes_beyond_its_array(model_layer):
    L = _lib.lib()
    T, k, H, I = 600, 8, model_layer.H, model_layer.I
    assert L.moe_workspace_bytes(T, k, model_layer.E, H, I) > (8 << 20)
    g, u, d = model_layer.gate.c(), model_layer.up.c(), model_layer.down.c()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the size check fails first
    st = L.nvfp4_expert_mlp_noalloc(fake, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), fake,
                                    fake, T, k, H, I, fake, None)
    assert st == -3
