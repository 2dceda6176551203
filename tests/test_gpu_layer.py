"""Whole-block GPU parity against the fp64 oracle on the seeded model-shaped
workloads (full size on the GPU; the oracle checks every token where it runs
in seconds and a sample of tokens at prefill sizes), plus determinism, graph
replay and small odd shapes."""
import math

import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import formats as F
from oracle import moe as M
from oracle.quantize import quantize_experts

import nvfp4_weight_only_moe_amd as moe
from nvfp4_weight_only_moe_amd import workload as W

from parity_util import (REL_FROB_TOL, OracleExperts, check_route, rel_frob, router_f64, row_rel)

pytestmark = pytest.mark.gpu

_LAYER = {}


@pytest.fixture(scope="module")
def layer0():
    assert torch.cuda.is_available()
    moe.lib()
    if "plain" not in _LAYER:
        _LAYER["plain"] = W.build_layer(0, zipf=False)
    return _LAYER["plain"]


@pytest.fixture(scope="module")
def layer0_zipf(layer0):
    if "zipf" not in _LAYER:
        p = S.router_params(0, zipf=True)
        wr, sc, pes, bias = W.router_to_device(p)
        _LAYER["zipf"] = moe.MoeLayer(wr, sc, pes, bias, layer0.gate, layer0.up, layer0.down, 8)
    return _LAYER["zipf"]


@pytest.fixture(scope="module")
def oracle_experts():
    return OracleExperts(0)


def _run(layer, x_bits):
    T = x_bits.shape[0]
    buf = moe.MoeBuffers(T, layer.H, layer.I, layer.E, layer.top_k)
    moe.forward(layer, W.to_device_bf16(x_bits), buf)
    torch.cuda.synchronize()
    return buf


def _check_block(buf, x_bits, router_p, oe, sample=None, tol=REL_FROB_TOL):
    T = x_bits.shape[0]
    r = router_f64(router_p)
    xs = F.bf16_bits_to_f64(x_bits)
    toks = np.arange(T) if sample is None else np.asarray(sample)
    ref_r = M.route(xs[toks], r["w_router"], r["scale"], r["per_expert_scale"], 8, r["bias"])
    gidx = buf.topk_idx.cpu().numpy()[toks]
    check_route(gidx, buf.topk_w.cpu().numpy()[toks], buf.topk_w_raw.cpu().numpy()[toks], ref_r,
                r["per_expert_scale"])
    assert buf.bucket_error_count() == 0
    oe.prefetch(np.unique(gidx))
    # the oracle follows the GPU's choice on flagged near-ties (same set otherwise)
    blk = M.moe_block(xs[toks], xs[toks], r, oe.fn(S.GATE), oe.fn(S.UP), oe.fn(S.DOWN), k=8,
                      ids=gidx.astype(np.int64))
    ref = blk["out"]
    got = buf.out.float().cpu().numpy()[toks]
    err = rel_frob(got, ref)
    assert np.all(np.isfinite(got))
    assert err <= tol, err
    # the expert output rows of these tokens' pairs, each against the oracle's
    # row of the same (token, slot): GPU rank from pair_rank, oracle rank from
    # its own bucketing of the sample (the four-call path: the decode path
    # keeps them on chip)
    if not buf.y_sorted_valid:
        return err, np.max(row_rel(got, ref))
    k = 8
    gpr = buf.pair_rank.cpu().numpy().reshape(-1, k)[toks].reshape(-1)
    y_got = buf.y_sorted[torch.from_numpy(gpr.astype(np.int64)).cuda()].float().cpu().numpy()
    y_ref = blk["y_sorted"][blk["buckets"]["pair_rank"]]
    assert np.all(np.isfinite(y_got))
    assert np.max(row_rel(y_got, y_ref)) <= tol
    return err, np.max(row_rel(got, ref))


def test_layer_T4_all_tokens(layer0, oracle_experts):
    x = S.activations(0, 4)
    buf = _run(layer0, x)
    err, worst_row = _check_block(buf, x, S.router_params(0), oracle_experts)
    assert worst_row <= 1e-2
    print(f"T=4 rel_frob={err:.3e} worst_row={worst_row:.3e}")


def test_layer_T64_all_tokens(layer0, oracle_experts):
    x = S.activations(1, 64)
    buf = _run(layer0, x)
    err, worst_row = _check_block(buf, x, S.router_params(0), oracle_experts)
    assert worst_row <= 1e-2
    print(f"T=64 rel_frob={err:.3e} worst_row={worst_row:.3e}")


@pytest.mark.parametrize("T", [16, 128])
def test_layer_decode_sizes_all_tokens(layer0, oracle_experts, T):
    # T = 16: GEMV with the K split; T = 128: 16-row GEMV tiles, unsplit
    x = S.activations(5, T)
    buf = _run(layer0, x)
    err, worst_row = _check_block(buf, x, S.router_params(0), oracle_experts)
    assert worst_row <= 1e-2
    print(f"T={T} rel_frob={err:.3e} worst_row={worst_row:.3e}")


@pytest.mark.parametrize("T", [24, 256, 512])
def test_layer_intermediate_T_zipf(layer0_zipf, oracle_experts, T):
    """Batched decode with skewed (Zipf) routing at token counts around the
    GEMV / GEMM crossover (fewer / more than 24 rows per active expert on
    average): every token for T = 24, a sample beyond."""
    x = S.activations(9, T)
    buf = _run(layer0_zipf, x)
    sample = None if T <= 64 else np.linspace(0, T - 1, 16).astype(int)
    err, _ = _check_block(buf, x, S.router_params(0, zipf=True), oracle_experts, sample)
    counts = np.diff(buf.expert_offsets.cpu().numpy())
    print(f"T={T} zipf rel_frob={err:.3e} rows/active expert={counts.sum() / max(1, (counts > 0).sum()):.1f}")


@pytest.mark.parametrize("T", [1, 8])
def test_layer_sweep_shapes_all_tokens(layer0, oracle_experts, T):
    """The per-layer shapes of the 30-layer decode sweep (T = 1: the split-K
    down GEMV; T = 8), every token."""
    x = S.activations(3, T)
    buf = _run(layer0, x)
    err, worst_row = _check_block(buf, x, S.router_params(0), oracle_experts)
    assert worst_row <= 1e-2
    print(f"T={T} rel_frob={err:.3e} worst_row={worst_row:.3e}")


def _check_sorted_rows(buf, ref_blk, rows=None, tol=REL_FROB_TOL):
    """Every (or the given) sorted expert output row of y_sorted against the
    oracle's, row by row (same bucketing: the ids are the GPU's)."""
    got = buf.y_sorted.float().cpu().numpy()
    ref = ref_blk["y_sorted"]
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(got))
    worst = float(np.max(row_rel(got, ref)))
    assert worst <= tol, worst
    return rel_frob(got, ref), worst


def test_layer_T2048_zipf_every_token(layer0_zipf, oracle_experts):
    """Prefill T = 2048 with Zipf routing: every token of the output and every
    sorted row of the expert outputs (all 16,384, covering every expert's
    ragged last row block) against the fp64 oracle."""
    x = S.activations(2, 2048)
    buf = _run(layer0_zipf, x)
    counts = np.diff(buf.expert_offsets.cpu().numpy())
    assert counts.sum() == 2048 * 8
    assert counts.max() > 4 * counts.mean()   # the skew is there
    r = router_f64(S.router_params(0, zipf=True))
    xs = F.bf16_bits_to_f64(x)
    ref_r = M.route(xs, r["w_router"], r["scale"], r["per_expert_scale"], 8, r["bias"])
    gidx = buf.topk_idx.cpu().numpy()
    check_route(gidx, buf.topk_w.cpu().numpy(), buf.topk_w_raw.cpu().numpy(), ref_r,
                r["per_expert_scale"])
    oracle_experts.prefetch(range(128))
    blk = M.moe_block(xs, xs, r, oracle_experts.fn(S.GATE), oracle_experts.fn(S.UP),
                      oracle_experts.fn(S.DOWN), k=8, ids=gidx.astype(np.int64))
    assert np.array_equal(buf.expert_offsets.cpu().numpy(), blk["buckets"]["offsets"])
    assert np.array_equal(buf.sorted_pairs.cpu().numpy(), blk["buckets"]["sorted_pairs"])
    ey, wy = _check_sorted_rows(buf, blk)
    got = buf.out.float().cpu().numpy()
    err = rel_frob(got, blk["out"])
    worst = float(np.max(row_rel(got, blk["out"])))
    assert err <= REL_FROB_TOL and worst <= REL_FROB_TOL, (err, worst)
    print(f"T=2048 all tokens rel_frob={err:.3e} worst_row={worst:.3e}; y_sorted rel_frob={ey:.3e} "
          f"worst_row={wy:.3e}; max/mean={counts.max() / counts.mean():.1f}")


def test_layer_T16384_zipf_outliers(layer0_zipf, oracle_experts):
    """Long prefill with 1% outlier rows (x20): all 164 outlier tokens and 256
    other tokens, checked separately (the outliers would otherwise dominate
    the norm), and their sorted expert rows."""
    x = S.activations(4, 16384, outliers=True)
    buf = _run(layer0_zipf, x)
    out_rows = S.outlier_rows(4, 16384)
    assert len(out_rows) == 164
    rng = np.random.default_rng(16384)
    normal = np.sort(rng.choice(np.setdiff1d(np.arange(16384), out_rows), 256, replace=False))
    e1, w1 = _check_block(buf, x, S.router_params(0, zipf=True), oracle_experts, out_rows)
    e2, w2 = _check_block(buf, x, S.router_params(0, zipf=True), oracle_experts, normal)
    assert w1 <= REL_FROB_TOL and w2 <= REL_FROB_TOL, (w1, w2)
    print(f"T=16384 outlier rows rel_frob={e1:.3e} worst={w1:.3e}; normal rows={e2:.3e} worst={w2:.3e}")


# ------------------------- sparse branch with its learned norms, layer step
def _branch_check(layer, x_bits, router_p, oe, T_sample=None, step=True, with_h1=True,
                  scalar=0.8, workload=6):
    """forward_branch against the oracle's sparse_branch ("Gemma 4 26B-A4B
    (MoE) - Core AI", Architecture code sketch).  Returns the relative error of
    the output and, for the layer step, of its normed part (out / scalar -
    residual), which the residual would otherwise dominate."""
    T = x_bits.shape[0]
    pre2, post2, post = S.norm_weights(0)
    norms = moe.BranchNorms(W.to_device_bf16(pre2), W.to_device_bf16(post2),
                            W.to_device_bf16(post) if step else None, 1e-6, scalar)
    h1_bits = S.dense_branch_output(workload, T) if (step and with_h1) else None
    buf = moe.MoeBuffers(T, layer.H, layer.I, layer.E, layer.top_k)
    x = W.to_device_bf16(x_bits)
    moe.forward_branch(layer, x, buf, norms,
                       h1=None if h1_bits is None else W.to_device_bf16(h1_bits))
    torch.cuda.synchronize()
    r = router_f64(router_p)
    xs = F.bf16_bits_to_f64(x_bits)
    toks = np.arange(T) if T_sample is None else np.asarray(T_sample)
    gidx = buf.topk_idx.cpu().numpy()[toks]
    ref_r = M.route(xs[toks], r["w_router"], r["scale"], r["per_expert_scale"], 8, r["bias"])
    check_route(gidx, buf.topk_w.cpu().numpy()[toks], buf.topk_w_raw.cpu().numpy()[toks], ref_r,
                r["per_expert_scale"])
    oe.prefetch(np.unique(gidx))
    f64 = F.bf16_bits_to_f64
    ref = M.sparse_branch(xs[toks], r, f64(pre2), f64(post2), oe.fn(S.GATE), oe.fn(S.UP),
                          oe.fn(S.DOWN), k=8, ids=gidx.astype(np.int64),
                          post_norm=f64(post) if step else None,
                          h1=None if h1_bits is None else f64(h1_bits)[toks], layer_scalar=scalar)
    got = buf.out.float().cpu().numpy()[toks]
    assert np.all(np.isfinite(got))
    if not step:
        return rel_frob(got, ref["h2"]), None
    return rel_frob(got, ref["out"]), rel_frob(got / scalar - xs[toks], ref["out"] / scalar - xs[toks])


@pytest.mark.parametrize("T", [4, 64])
def test_branch_with_norms_all_tokens(layer0, oracle_experts, T):
    x = S.activations(6, T)
    err_out, err_part = _branch_check(layer0, x, S.router_params(0), oracle_experts)
    assert err_out <= REL_FROB_TOL and err_part <= REL_FROB_TOL, (err_out, err_part)
    # h1 = 0 (no dense branch)
    e0, p0 = _branch_check(layer0, x, S.router_params(0), oracle_experts, with_h1=False)
    assert e0 <= REL_FROB_TOL and p0 <= REL_FROB_TOL, (e0, p0)
    # without the outer norm the output is h2, the sparse branch alone
    eb, _ = _branch_check(layer0, x, S.router_params(0), oracle_experts, step=False)
    assert eb <= REL_FROB_TOL, eb
    print(f"T={T} layer step: out {err_out:.3e}, normed part {err_part:.3e}; h1 = 0 {p0:.3e}; "
          f"h2 alone {eb:.3e}")


def test_branch_with_norms_prefill_sampled(layer0_zipf, oracle_experts):
    x = S.activations(7, 2048)
    sample = np.linspace(0, 2047, 10).astype(int)
    e, part = _branch_check(layer0_zipf, x, S.router_params(0, zipf=True), oracle_experts, sample,
                            workload=7)
    assert e <= REL_FROB_TOL and part <= REL_FROB_TOL, (e, part)
    eb, _ = _branch_check(layer0_zipf, x, S.router_params(0, zipf=True), oracle_experts, sample,
                          step=False)
    assert eb <= REL_FROB_TOL, eb


def test_chained_layers_teacher_forced():
    """Three layers chained through the residual (layer l reads layer l-1's
    bf16 output; the dense branch absent, h1 = 0), each layer checked against
    the oracle's layer step on the input the GPU actually gave it."""
    T, scalar = 4, 0.9
    x_bits = S.activations(8, T)
    x = W.to_device_bf16(x_bits)
    f64 = F.bf16_bits_to_f64
    for l in range(3):
        layer = W.build_layer(l, zipf=False)
        pre2, post2, post = S.norm_weights(l)
        norms = moe.BranchNorms(*[W.to_device_bf16(a) for a in (pre2, post2, post)], 1e-6, scalar)
        buf = moe.MoeBuffers(T, layer.H, layer.I, layer.E, layer.top_k)
        moe.forward_branch(layer, x, buf, norms)
        torch.cuda.synchronize()
        xin = f64(x.view(torch.int16).cpu().numpy().view(np.uint16))
        r = router_f64(S.router_params(l))
        gidx = buf.topk_idx.cpu().numpy()
        ref_r = M.route(xin, r["w_router"], r["scale"], r["per_expert_scale"], 8, r["bias"])
        check_route(gidx, buf.topk_w.cpu().numpy(), buf.topk_w_raw.cpu().numpy(), ref_r,
                    r["per_expert_scale"])
        oe = OracleExperts(l)
        oe.prefetch(np.unique(gidx))
        ref = M.sparse_branch(xin, r, f64(pre2), f64(post2), oe.fn(S.GATE), oe.fn(S.UP),
                              oe.fn(S.DOWN), k=8, ids=gidx.astype(np.int64), post_norm=f64(post),
                              layer_scalar=scalar)
        got = buf.out.float().cpu().numpy()
        assert rel_frob(got, ref["out"]) <= REL_FROB_TOL
        assert rel_frob(got / scalar - xin, ref["out"] / scalar - xin) <= REL_FROB_TOL
        x = buf.out.clone()
        del layer
        torch.cuda.empty_cache()


def test_layer_deterministic(layer0):
    x = S.activations(1, 64)
    a = _run(layer0, x)
    b = _run(layer0, x)
    for name in ("topk_idx", "topk_w", "expert_offsets", "sorted_pairs", "pair_rank", "y_sorted", "out"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_graph_replay_matches_eager(layer0):
    x = W.to_device_bf16(S.activations(1, 64))
    eager = moe.MoeBuffers(64, layer0.H, layer0.I, layer0.E, 8)
    moe.forward(layer0, x, eager)
    buf = moe.MoeBuffers(64, layer0.H, layer0.I, layer0.E, 8)
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
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf.out, eager.out)
        assert torch.equal(buf.sorted_pairs, eager.sorted_pairs)


def test_graph_replay_matches_eager_prefill(layer0_zipf):
    """The prefill path in a graph (wide router, multi-kernel bucketing,
    tiled GEMMs): every replay, with eager work between them, equals eager."""
    x = W.to_device_bf16(S.activations(2, 2048))
    eager = moe.MoeBuffers(2048, layer0_zipf.H, layer0_zipf.I, layer0_zipf.E, 8)
    moe.forward(layer0_zipf, x, eager)
    buf = moe.MoeBuffers(2048, layer0_zipf.H, layer0_zipf.I, layer0_zipf.E, 8)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(layer0_zipf, x, buf)     # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(layer0_zipf, x, buf)
    for _ in range(3):
        buf.out.zero_()
        buf.expert_offsets.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf.out, eager.out)
        assert torch.equal(buf.expert_offsets, eager.expert_offsets)
        assert torch.equal(buf.sorted_pairs, eager.sorted_pairs)


@pytest.mark.parametrize("T", [5, 300])
def test_separate_expert_input(T):
    """forward with an expert input other than the router's x (moe_route_bucket
    + nvfp4_expert_mlp + moe_combine): the experts read x_expert, the router x."""
    T, k, E, H, I = T, 4, 16, 192, 128
    c = S.small_case(40 + T, T, H, I, E, k)
    xe_bits = S.small_case(41 + T, T, H, I, E, k)["x"]
    layer = W.build_small_layer(c, k)
    buf = moe.MoeBuffers(T, H, I, E, k)
    moe.forward(layer, W.to_device_bf16(c["x"]), buf, x_expert=W.to_device_bf16(xe_bits))
    torch.cuda.synchronize()
    r = router_f64(c["router"])
    xs, xe = F.bf16_bits_to_f64(c["x"]), F.bf16_bits_to_f64(xe_bits)
    ref_r = M.route(xs, r["w_router"], r["scale"], r["per_expert_scale"], k, r["bias"])
    gidx = buf.topk_idx.cpu().numpy()
    check_route(gidx, buf.topk_w.cpu().numpy(), buf.topk_w_raw.cpu().numpy(), ref_r,
                r["per_expert_scale"])
    q = {n: quantize_experts(F.bf16_bits_to_f64(c[n])) for n in ("gate", "up", "down")}
    fns = {n: M.nvfp4_weights(*q[n]) for n in q}
    ref = M.moe_block(xs, xe, r, fns["gate"], fns["up"], fns["down"], k=k, ids=gidx)["out"]
    got = buf.out.float().cpu().numpy()
    assert rel_frob(got, ref) <= REL_FROB_TOL
    # and not what the router's x would have given
    wrong = M.moe_block(xs, xs, r, fns["gate"], fns["up"], fns["down"], k=k, ids=gidx)["out"]
    assert rel_frob(got, wrong) > 0.5


@pytest.mark.parametrize("T,k,E,H,I,zipf", [(1, 2, 16, 128, 64, False), (3, 2, 16, 128, 64, False),
                                            (5, 4, 32, 192, 128, True), (50, 8, 16, 256, 64, True)])
def test_small_block_odd_shapes(T, k, E, H, I, zipf):
    c = S.small_case(T * 7 + E, T, H, I, E, k, zipf)
    layer = W.build_small_layer(c, k)
    buf = moe.MoeBuffers(T, H, I, E, k)
    moe.forward(layer, W.to_device_bf16(c["x"]), buf)
    torch.cuda.synchronize()
    r = router_f64(c["router"])
    xs = F.bf16_bits_to_f64(c["x"])
    ref_r = M.route(xs, r["w_router"], r["scale"], r["per_expert_scale"], k, r["bias"])
    gidx = buf.topk_idx.cpu().numpy()
    check_route(gidx, buf.topk_w.cpu().numpy(), buf.topk_w_raw.cpu().numpy(), ref_r,
                r["per_expert_scale"])
    q = {n: quantize_experts(F.bf16_bits_to_f64(c[n])) for n in ("gate", "up", "down")}
    fns = {n: M.nvfp4_weights(*q[n]) for n in q}
    ref = M.moe_block(xs, xs, r, fns["gate"], fns["up"], fns["down"], k=k, ids=gidx)["out"]
    dense = M.moe_block_dense(xs, xs, r, fns["gate"], fns["up"], fns["down"], k=k)
    got = buf.out.float().cpu().numpy()
    assert rel_frob(got, ref) <= REL_FROB_TOL
    if np.array_equal(np.sort(gidx, 1), np.sort(ref_r["idx"], 1)):
        assert rel_frob(got, dense) <= REL_FROB_TOL


def test_empty_batch_is_noop(layer0):
    buf = moe.MoeBuffers(0, layer0.H, layer0.I, layer0.E, 8)
    moe.forward(layer0, torch.empty((0, layer0.H), dtype=torch.bfloat16, device="cuda"), buf)
    torch.cuda.synchronize()
    assert buf.expert_offsets.cpu().numpy().tolist() == [0] * (layer0.E + 1)
