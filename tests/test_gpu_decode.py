"""moe_layer_decode (the whole block of a decode batch in three or four
launches) against the four-call path and the fp64 oracle: every routing and
bucketing byte equal to the four calls', the output too above 32 pairs and
within a bf16 step of it up to 32 pairs (down and combine in one kernel, which
packs each expert's row differently in the matrix core), and within the block
bar of the oracle, on model shapes (T = 1 .. 8) and small odd shapes, in every
weight format, in a graph."""
import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import formats as F
from oracle import int4 as Q
from oracle import moe as M
from oracle.quantize import quantize_experts

import nvfp4_weight_only_moe_amd as moe
from nvfp4_weight_only_moe_amd import _lib
from nvfp4_weight_only_moe_amd import workload as W

from parity_util import (REL_FROB_TOL, OracleExperts, check_route, rel_frob, router_f64, row_rel)

pytestmark = pytest.mark.gpu

_L = {}
# decode batches of up to this many pairs run down and the combine as one kernel
FUSED_COMBINE_MAX_P = 32


@pytest.fixture(scope="module")
def layer0():
    assert torch.cuda.is_available()
    moe.lib()
    if "l0" not in _L:
        _L["l0"] = W.build_layer(0)
    return _L["l0"]


@pytest.fixture(scope="module")
def oe():
    return OracleExperts(0)


def _both(layer, x_bits):
    """The block through moe_layer_decode and through the four calls."""
    T = x_bits.shape[0]
    x = W.to_device_bf16(x_bits)
    a = moe.MoeBuffers(T, layer.H, layer.I, layer.E, layer.top_k)
    b = moe.MoeBuffers(T, layer.H, layer.I, layer.E, layer.top_k)
    assert a.decode
    moe.forward(layer, x, a, fused=True)
    moe.forward(layer, x, b, fused=False)
    torch.cuda.synchronize()
    for name in ("topk_idx", "topk_w", "topk_w_raw", "expert_offsets", "sorted_pairs", "pair_rank"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    if T * layer.top_k > FUSED_COMBINE_MAX_P:
        assert torch.equal(a.out, b.out)
    else:
        # each expert output Y may differ by its last bf16 bit: the sum by a
        # few bf16 steps at most, relative to the row
        ga, gb = a.out.float(), b.out.float()
        row = gb.abs().amax(dim=1, keepdim=True).clamp_min(1e-30)
        assert float(((ga - gb).abs() / row).max()) <= 2 ** -6
        assert rel_frob(ga.cpu().numpy(), gb.cpu().numpy()) <= 2e-3
    assert a.bucket_error_count() == 0
    return a, b


def _oracle_out(layer_router, x_bits, gidx, fns, k):
    r = router_f64(layer_router)
    xs = F.bf16_bits_to_f64(x_bits)
    ref_r = M.route(xs, r["w_router"], r["scale"], r["per_expert_scale"], k, r["bias"])
    return r, ref_r, M.moe_block(xs, xs, r, *fns, k=k, ids=gidx.astype(np.int64))["out"]


@pytest.mark.parametrize("T", [1, 2, 4, 7, 8])
def test_layer_decode_model_shape(layer0, oe, T):
    x = S.activations(30 + T, T)
    a, b = _both(layer0, x)
    gidx = a.topk_idx.cpu().numpy()
    oe.prefetch(np.unique(gidx))
    r, ref_r, ref = _oracle_out(S.router_params(0), x, gidx,
                                (oe.fn(S.GATE), oe.fn(S.UP), oe.fn(S.DOWN)), 8)
    check_route(gidx, a.topk_w.cpu().numpy(), a.topk_w_raw.cpu().numpy(), ref_r,
                r["per_expert_scale"])
    got = a.out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    err, worst = rel_frob(got, ref), float(np.max(row_rel(got, ref)))
    assert err <= REL_FROB_TOL and worst <= REL_FROB_TOL, (err, worst)
    print(f"T={T} fused rel_frob={err:.3e} worst_row={worst:.3e}")


@pytest.mark.parametrize("T,k,E,H,I,zipf", [(1, 2, 16, 128, 64, False), (3, 4, 16, 192, 128, True),
                                            (8, 8, 32, 256, 192, False), (5, 3, 16, 4096, 64, True),
                                            (8, 8, 256, 128, 64, False), (2, 16, 32, 64, 128, False)])
def test_layer_decode_small_shapes(T, k, E, H, I, zipf):
    c = S.small_case(500 + T * 7 + E, T, H, I, E, k, zipf)
    layer = W.build_small_layer(c, k)
    a, b = _both(layer, c["x"])
    q = {n: quantize_experts(F.bf16_bits_to_f64(c[n])) for n in ("gate", "up", "down")}
    fns = {n: M.nvfp4_weights(*q[n]) for n in q}
    gidx = a.topk_idx.cpu().numpy()
    r, ref_r, ref = _oracle_out(c["router"], c["x"], gidx, (fns["gate"], fns["up"], fns["down"]), k)
    check_route(gidx, a.topk_w.cpu().numpy(), a.topk_w_raw.cpu().numpy(), ref_r,
                r["per_expert_scale"])
    got = a.out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert rel_frob(got, ref) <= REL_FROB_TOL
    assert np.max(row_rel(got, ref)) <= REL_FROB_TOL


def _int4_fn(fmt, stack):
    packed, sb = stack

    def get(e):
        bits = sb[e].view(np.uint16)
        if fmt == "q4_0":
            return Q.decode_q4_0(packed[e], bits)
        return Q.decode_aff4(packed[e], bits.reshape(bits.shape[0], -1, 2))
    return get


@pytest.mark.parametrize("fmt_gu,fmt_d", [("q4_0", "q4_0"), ("aff4", "aff4"), ("q4_0", "aff4")])
def test_layer_decode_int4_formats(fmt_gu, fmt_d):
    T, k, E, H, I = 6, 4, 16, 256, 128
    c = S.small_int4_case(77, fmt_gu, T, H, I, E, k)
    if fmt_d != fmt_gu:
        c["down"] = S.small_int4_case(77, fmt_d, T, H, I, E, k)["down"]
    wr, sc, pes, bias = W.router_to_device(c["router"])
    g, u = (W.int4_to_device(fmt_gu, *c[n]) for n in ("gate", "up"))
    d = W.int4_to_device(fmt_d, *c["down"])
    layer = moe.MoeLayer(wr, sc, pes, bias, g, u, d, k)
    a, b = _both(layer, c["x"])
    gidx = a.topk_idx.cpu().numpy()
    fns = (_int4_fn(fmt_gu, c["gate"]), _int4_fn(fmt_gu, c["up"]), _int4_fn(fmt_d, c["down"]))
    _, _, ref = _oracle_out(c["router"], c["x"], gidx, fns, k)
    got = a.out.float().cpu().numpy()
    assert rel_frob(got, ref) <= REL_FROB_TOL
    assert np.max(row_rel(got, ref)) <= REL_FROB_TOL


@pytest.mark.parametrize("fmt", ["q4_0", "aff4"])
def test_layer_decode_int4_model_shape(fmt):
    """The int4 formats through moe_layer_decode at the model's shape, where
    from 4 tokens on the gate/up kernel takes three row-tile pairs per wave
    (15 column groups of 48, the last one partly past I = 704): every routing
    byte and the output equal to the four calls (T = 8), within a bf16 step
    (T = 4: down and combine in one kernel)."""
    key = f"int4_{fmt}"
    if key not in _L:
        _L[key] = W.build_int4_layer(fmt, 0)
    for T in (4, 8):
        _both(_L[key], S.activations(50 + T, T))


@pytest.mark.parametrize("T", [2, 8])
def test_layer_decode_deterministic_and_graph_replay(layer0, T):
    x = W.to_device_bf16(S.activations(40, T))
    eager = moe.MoeBuffers(T, layer0.H, layer0.I, layer0.E, 8)
    moe.forward(layer0, x, eager)
    again = moe.MoeBuffers(T, layer0.H, layer0.I, layer0.E, 8)
    moe.forward(layer0, x, again)
    torch.cuda.synchronize()
    assert torch.equal(eager.out, again.out)
    buf = moe.MoeBuffers(T, layer0.H, layer0.I, layer0.E, 8)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(layer0, x, buf)          # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(layer0, x, buf)
    for _ in range(3):
        buf.out.zero_()
        buf.expert_offsets.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf.out, eager.out)
        assert torch.equal(buf.expert_offsets, eager.expert_offsets)
