"""Pins of the oracle's router, bucketing, experts and whole block (CPU only):
torch library routines, closed forms, invariants, the dense over-read
formulation on tiny shapes, and the model dimensions the pages print."""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import formats as F
from oracle import moe as M
from oracle.quantize import quantize_experts
import moe_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(bits):
    return F.bf16_bits_to_f64(bits)


def _small(t=5, h=32, i=16, e=8, k=2, seed=0, zipf=False):
    c = S.small_case(seed, t, h, i, e, k, zipf)
    router = dict(w_router=_f64(c["router"]["w_router"]), scale=_f64(c["router"]["scale"]),
                  per_expert_scale=_f64(c["router"]["per_expert_scale"]), bias=c["router"]["bias"])
    q = {n: quantize_experts(_f64(c[n])) for n in ("gate", "up", "down")}
    fns = {n: M.nvfp4_weights(*q[n]) for n in q}
    return _f64(c["x"]), router, fns


def test_gelu_tanh_vs_torch():
    x = np.linspace(-12, 12, 10001)
    ref = TF.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(M.gelu_tanh(x) - ref)) <= 1e-15


def test_router_vs_torch_library_routines():
    x, router, _ = _small(t=9, h=64, e=16, k=4, seed=1)
    r = M.route(x, router["w_router"], router["scale"], router["per_expert_scale"], k=4)
    xt = torch.from_numpy(x)
    n = TF.rms_norm(xt, (64,), eps=1e-6)
    logits = TF.linear(n * torch.from_numpy(router["scale"]) * 64 ** -0.5,
                       torch.from_numpy(router["w_router"]))
    p = TF.softmax(logits, dim=-1)
    top_p, top_i = torch.topk(p, 4, dim=-1)
    w_raw = top_p / top_p.sum(-1, keepdim=True)
    w = w_raw * torch.from_numpy(router["per_expert_scale"])[top_i]
    assert np.max(np.abs(r["logits"] - logits.numpy())) < 1e-13
    for ti in range(9):
        assert set(r["idx"][ti].tolist()) == set(top_i[ti].tolist())
        order_o = np.argsort(r["idx"][ti])
        order_t = np.argsort(top_i[ti].numpy())
        assert np.allclose(r["w"][ti][order_o], w[ti].numpy()[order_t], atol=1e-14, rtol=0)
        assert np.allclose(r["w_raw"][ti][order_o], w_raw[ti].numpy()[order_t], atol=1e-14, rtol=0)


def test_router_invariants_full_size():
    p = S.router_params(0)
    x = _f64(S.activations(1, 64))
    wr, sc, pes = _f64(p["w_router"]), _f64(p["scale"]), _f64(p["per_expert_scale"])
    r = M.route(x, wr, sc, pes, k=8)
    assert np.max(np.abs(r["w_raw"].sum(1) - 1.0)) <= 1e-12
    full = np.argsort(-r["logits"], axis=1, kind="stable")[:, :8]
    for ti in range(64):
        assert set(full[ti].tolist()) == set(r["idx"][ti].tolist())
    # w_raw is the softmax over the selected logits (closed form)
    sel = np.take_along_axis(r["logits"], r["idx"], 1)
    ref = np.exp(sel - sel.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.max(np.abs(ref - r["w_raw"])) <= 1e-14
    # scale-freeness: x * 4 is exact in bf16; only eps moves the logits
    r4 = M.route(x * 4.0, wr, sc, pes, k=8)
    for ti in range(64):
        if not r["near_tie"][ti]:
            assert set(r4["idx"][ti].tolist()) == set(r["idx"][ti].tolist())
    assert np.max(np.abs(r4["logits"] - r["logits"])) < 1e-7


def test_topk_tie_goes_to_lower_id():
    logits = np.array([[0.0, 1.0, 1.0, 1.0, 0.5]])
    assert M.topk_ids(logits, 2).tolist() == [[1, 2]]
    assert M.topk_ids(np.zeros((1, 6)), 3).tolist() == [[0, 1, 2]]


def test_zero_row_routes_to_first_experts():
    x = np.zeros((1, 32))
    r = M.route(x, np.ones((8, 32)), np.ones(32), np.ones(8), k=3)
    assert r["idx"].tolist() == [[0, 1, 2]]
    assert np.allclose(r["w_raw"], 1 / 3)


def test_bucket_properties():
    rng = np.random.default_rng(3)
    idx = np.stack([rng.choice(16, 4, replace=False) for _ in range(37)])
    b = M.bucket(idx, 16)
    assert np.array_equal(b["counts"], np.bincount(idx.reshape(-1), minlength=16))
    assert b["offsets"][0] == 0 and b["offsets"][-1] == idx.size
    assert np.all(np.diff(b["offsets"]) >= 0)
    sp = b["sorted_pairs"]
    assert sorted(sp.tolist()) == list(range(idx.size))
    flat = idx.reshape(-1)
    for e in range(16):
        seg = sp[b["offsets"][e]:b["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    assert np.array_equal(sp[b["pair_rank"]], np.arange(idx.size))


def test_experts_plain_gemm_special_case():
    # all block scales 1.0 (code 0x38) and g = 1: the dequantised weights are
    # the E2M1 values, so the expert is a plain GEMM chain (torch fp64)
    rng = np.random.default_rng(4)
    codes = {n: rng.integers(0, 16, size=s).astype(np.uint8)
             for n, s in (("g", (16, 64)), ("u", (16, 64)), ("d", (64, 16)))}
    w = {n: F.dequantize(F.pack_nibbles(c), np.full((c.shape[0], c.shape[1] // 16), 0x38, np.uint8), 1.0)
         for n, c in codes.items()}
    x = rng.standard_normal((5, 64))
    y = M.expert_mlp(x, w["g"], w["u"], w["d"])
    xt = torch.from_numpy(x)
    tw = {n: torch.from_numpy(F.e2m1_decode(c)) for n, c in codes.items()}
    ref = (TF.gelu(xt @ tw["g"].T, approximate="tanh") * (xt @ tw["u"].T)) @ tw["d"].T
    assert np.max(np.abs(y - ref.numpy())) <= 1e-14 * np.abs(ref.numpy()).max()


@pytest.mark.parametrize("t,zipf", [(1, False), (3, False), (5, True)])
def test_block_vs_dense_over_read(t, zipf):
    x, router, fns = _small(t=t, seed=t, zipf=zipf)
    a = M.moe_block(x, x, router, fns["gate"], fns["up"], fns["down"], k=2)["out"]
    b = M.moe_block_dense(x, x, router, fns["gate"], fns["up"], fns["down"], k=2)
    assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.abs(b).max())


def test_single_expert_is_plain_geglu_times_pes():
    x, router, fns = _small(t=4, e=1, k=1, seed=2)
    out = M.moe_block(x, x, router, fns["gate"], fns["up"], fns["down"], k=1)["out"]
    ref = M.expert_mlp(x, fns["gate"](0), fns["up"](0), fns["down"](0)) * router["per_expert_scale"][0]
    assert np.max(np.abs(out - ref)) <= 1e-13


def test_k_equals_e_is_dense_softmax_mixture():
    x, router, fns = _small(t=3, e=4, k=4, seed=5)
    router = dict(router, per_expert_scale=np.ones(4))
    out = M.moe_block(x, x, router, fns["gate"], fns["up"], fns["down"], k=4)["out"]
    p = M.softmax(M.router_logits(x, router["w_router"], router["scale"]))
    ref = sum(p[:, e:e + 1] * M.expert_mlp(x, fns["gate"](e), fns["up"](e), fns["down"](e))
              for e in range(4))
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_model_dims_and_printed_sizes():
    d = {l.split()[0]: float(l.split()[1]) for l in open(os.path.join(GOLDEN, "model_dims.txt"))
         if l.strip() and not l.startswith("#")}
    assert (S.H, S.E, S.TOP_K, S.I, S.LAYERS) == (d["hidden_size"], d["num_experts"], d["top_k"],
                                                  d["moe_intermediate_size"], d["num_layers"])
    assert S.GROUP == d["block_size"] and F.E2M1_MAX == d["e2m1_vmax"]
    params = S.LAYERS * S.E * 3 * S.I * S.H
    assert params == 22_837_985_280
    assert round(params / 1e9, 2) == d["routed_expert_params_G"]
    router_bytes = S.LAYERS * (S.E * S.H + S.H + S.E) * 2
    assert round(router_bytes / 1e9, 2) == d["router_set_GB"]


def test_synth_shapes_and_determinism():
    a = S.expert_weight(0, S.GATE, 3)
    b = S.expert_weight(0, S.GATE, 3)
    assert a.shape == (704, 2816) and np.array_equal(a, b)
    assert S.expert_weight(0, S.DOWN, 3).shape == (2816, 704)
    x = S.activations(4, 300, outliers=True)
    rows = S.outlier_rows(4, 300)
    assert len(rows) == 3
    base = S.activations(4, 300, outliers=False)
    assert np.array_equal(np.delete(x, rows, 0), np.delete(base, rows, 0))


# ------------------------------------------------ learned norms (NEXT-1)
def test_rms_norm_vs_torch_library_routine():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 96)) * rng.uniform(0.1, 30.0, (5, 1))
    w = rng.uniform(0.5, 1.5, 96)
    got = M.rms_norm(x, w, 1e-6)
    ref = TF.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_rms_norm_closed_forms():
    w = np.linspace(0.5, 2.0, 64)
    # a constant row c: every element is c / sqrt(c^2 + eps) * w
    for c in (3.0, -0.25):
        got = M.rms_norm(np.full((1, 64), c), w, 1e-6)[0]
        assert np.allclose(got, c / math.sqrt(c * c + 1e-6) * w, rtol=0, atol=1e-15)
    # scale-free when eps = 0; the output has root-mean-square |w|_rms for w = const
    x = np.random.default_rng(3).standard_normal((4, 64))
    assert np.allclose(M.rms_norm(7.5 * x, w, 0.0), M.rms_norm(x, w, 0.0), rtol=1e-14, atol=0)
    y = M.rms_norm(x, np.full(64, 2.0), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 2.0, rtol=1e-14)
    # a zero row stays zero (eps keeps it finite)
    assert np.all(M.rms_norm(np.zeros((1, 64)), w, 1e-6) == 0.0)


def _branch_case(seed=11, t=4, h=32, i=16, e=8, k=2):
    c = S.small_case(seed, t, h, i, e, k)
    r = {n: (F.bf16_bits_to_f64(v) if v is not None and n != "bias" else v)
         for n, v in c["router"].items()}
    x = F.bf16_bits_to_f64(c["x"])
    fn = {n: (lambda m: (lambda ex: F.bf16_bits_to_f64(m[ex])))(c[n]) for n in ("gate", "up", "down")}
    return x, r, fn


def test_layer_step_outer_norm_sees_h1_plus_h2():
    """"Gemma 4 26B-A4B (MoE) - Core AI", Architecture code sketch: the layer
    adds the residual to post_feedforward_layernorm(h1 + h2), then scales by
    layer_scalar.  Special cases with eps = 0, where the norms have closed
    forms, each failing for a plausible wrong composition."""
    x, r, fn = _branch_case()
    h, ones = x.shape[1], np.ones(x.shape[1])

    def step(**kw):
        base = dict(pre_norm2=ones, post_norm2=ones, post_norm=ones, eps=0.0)
        base.update(kw)
        # the expert input here is rms_norm(x, 1) (pre-norm weight one), not x
        return M.sparse_branch(x, r, base.pop("pre_norm2"), base.pop("post_norm2"), fn["gate"],
                               fn["up"], fn["down"], k=2, **base)

    # the pre-norm of the expert input is scale-free, so feed the block x / rms(x)
    s_n = M.moe_block(x, x / np.sqrt(np.mean(x * x, axis=1, keepdims=True)), r, fn["gate"],
                      fn["up"], fn["down"], k=2, eps=0.0)["out"]
    unit = s_n / np.sqrt(np.mean(s_n * s_n, axis=1, keepdims=True))
    # h1 = 0, outer weight 2: the outer norm of a unit-RMS row is 2x the row
    # (a missing outer norm, or the old residual + post_norm_2(sum), gives 1x)
    got = step(post_norm=np.full(h, 2.0))["out"]
    assert np.allclose(got, x + 2.0 * unit, rtol=0, atol=1e-12)
    # h1 = h2 (both unit RMS): norm(2 h2) = h2, so out = x + w * h2; adding h1
    # after the outer norm instead would give x + h2 + w * h2
    w = np.linspace(0.5, 1.5, h)
    got = step(post_norm=w, h1=unit)["out"]
    assert np.allclose(got, x + w * unit, rtol=0, atol=1e-12)
    # h1 = -h2 (the branch's own h2): the outer norm sees zero and the
    # residual passes alone, scaled (eps > 0 keeps the zero row finite)
    h2 = step(post_norm=None, eps=1e-6)["h2"]
    got = step(h1=-h2, layer_scalar=0.75, eps=1e-6)["out"]
    assert np.array_equal(got, 0.75 * x)
    # any h1: (out / scalar - residual) / w has RMS exactly 1 in every row
    h1 = np.random.default_rng(5).standard_normal(x.shape)
    got = step(post_norm=w, h1=h1, layer_scalar=0.5)["out"]
    v = (got / 0.5 - x) / w
    assert np.allclose(np.sqrt(np.mean(v * v, axis=1)), 1.0, rtol=1e-12)
    # the layer scalar multiplies the whole step (a power of two: exact)
    a = step(post_norm=w, h1=h1, layer_scalar=1.0)["out"]
    assert np.array_equal(step(post_norm=w, h1=h1, layer_scalar=0.25)["out"], 0.25 * a)
    # without the outer norm weight the step is not taken: h2 alone
    b = step(post_norm=None)
    assert b["out"] is None and np.allclose(b["h2"], unit, rtol=0, atol=1e-12)


def test_routing_reads_the_raw_residual_and_experts_the_normed_one():
    """Same sketch: router(residual) on the raw residual, the experts on
    pre_feedforward_layernorm_2(residual).  A per-channel pre-norm weight that
    reroutes the normed input shows which one the router read."""
    x, r, fn = _branch_case(seed=12, t=6, e=8, k=2)
    h = x.shape[1]
    pre = np.where(np.arange(h) % 2 == 0, 0.05, 4.0)
    raw = M.route(x, r["w_router"], r["scale"], r["per_expert_scale"], 2)["idx"]
    normed = M.route(M.rms_norm(x, pre), r["w_router"], r["scale"], r["per_expert_scale"], 2)["idx"]
    assert not np.array_equal(np.sort(raw, 1), np.sort(normed, 1))   # the pin can fail
    sb = M.sparse_branch(x, r, pre, np.ones(h), fn["gate"], fn["up"], fn["down"], k=2,
                         post_norm=np.ones(h))
    assert np.array_equal(np.sort(sb["block"]["route"]["idx"], 1), np.sort(raw, 1))
    # the experts read a scale-free norm of the residual: 4x (exact in fp64)
    # gives the same branch output h2 (eps = 0); the GELU-gated experts on
    # the raw residual would not be homogeneous in it
    a = M.sparse_branch(x, r, pre, np.ones(h), fn["gate"], fn["up"], fn["down"], k=2, eps=0.0)
    b = M.sparse_branch(4.0 * x, r, pre, np.ones(h), fn["gate"], fn["up"], fn["down"], k=2, eps=0.0)
    assert np.allclose(a["h2"], b["h2"], rtol=0, atol=1e-12)
    raw_in = M.moe_block(4.0 * x, 4.0 * x, r, fn["gate"], fn["up"], fn["down"], k=2, eps=0.0)["out"]
    raw_in1 = M.moe_block(x, x, r, fn["gate"], fn["up"], fn["down"], k=2, eps=0.0)["out"]
    assert not np.allclose(M.rms_norm(raw_in, np.ones(h), 0.0), M.rms_norm(raw_in1, np.ones(h), 0.0),
                           rtol=0, atol=1e-6)


def test_weights_for_ids_hand_computed():
    """Softmax probabilities at the given ids, renormalised over them, times
    per_expert_scale ("Gemma 4 26B-A4B (MoE) - Core AI", router description).
    logits ln(1, 2, 3, 4, 6): probabilities 1/16 .. 6/16; ids (4, 1) take
    6/16 and 2/16 -> 3/4 and 1/4 (renormalising the logits instead would give
    ln 6 / ln 12 = 0.72)."""
    logits = np.log(np.array([[1.0, 2.0, 3.0, 4.0, 6.0], [5.0, 5.0, 5.0, 5.0, 5.0]]))
    pes = np.array([1.0, 0.5, 2.0, 1.0, 1.5])
    ids = np.array([[4, 1], [2, 0]])
    w, w_raw = M.weights_for_ids(logits, pes, ids)
    assert np.allclose(w_raw, [[0.75, 0.25], [0.5, 0.5]], rtol=0, atol=1e-15)
    assert np.allclose(w, [[1.125, 0.125], [1.0, 0.5]], rtol=0, atol=1e-15)


def test_weights_for_ids_agrees_with_route():
    p = S.router_params(0)
    x = _f64(S.activations(1, 16))
    wr, sc, pes = _f64(p["w_router"]), _f64(p["scale"]), _f64(p["per_expert_scale"])
    r = M.route(x, wr, sc, pes, k=8)
    w, w_raw = M.weights_for_ids(r["logits"], pes, r["idx"])
    assert np.array_equal(w, r["w"]) and np.array_equal(w_raw, r["w_raw"])
    # a permutation of the ids permutes the weights
    perm = r["idx"][:, ::-1]
    w2, _ = M.weights_for_ids(r["logits"], pes, perm)
    assert np.allclose(w2, r["w"][:, ::-1], rtol=1e-15, atol=0)
