"""GPU parity of each C-ABI call against the oracle on the same seeded inputs.

Bit-exact: quantiser bytes, the bf16 decode, expert ids (outside near-ties),
bucketing.  Floating point: routing weights within 4e-6; expert outputs and
the combine within the bounds stated per test."""
import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import formats as F
from oracle import moe as M
from oracle.quantize import quantize, quantize_experts

import nvfp4_weight_only_moe_amd as moe
from nvfp4_weight_only_moe_amd import workload as W

from parity_util import (REL_FROB_TOL, check_route, rel_frob, router_f64, row_rel)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()  # raises if the HIP library is missing
    yield


def _bits(a):
    return W.to_device_bf16(a)


def _np_bf16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ---------------------------------------------------------------- quantiser
@pytest.mark.parametrize("shape", [(3, 48, 128), (2, 704, 2816), (2, 2816, 704)])
def test_quantize_bit_exact(shape):
    E, N, K = shape
    rng = np.random.default_rng(N)
    bits = S.f32_to_bf16_bits((rng.standard_normal(shape) * 0.02).astype(np.float32))
    bits[0, :, 16:32] = 0                      # an all-zero block column
    out = moe.Nvfp4Weights.empty(E, N, K)
    moe.nvfp4_quantize(_bits(bits), out)
    torch.cuda.synchronize()
    p, s, g = quantize_experts(F.bf16_bits_to_f64(bits))
    assert np.array_equal(out.packed.cpu().numpy(), p)
    assert np.array_equal(out.scales.cpu().numpy(), s)
    assert np.array_equal(out.global_scale.cpu().numpy().astype(np.float64), g)


def test_quantize_edge_tensors():
    # zero tensor, on-grid tensor (g = 1, scales 448), tiny values (subnormal
    # E4M3 block scales) and exact E2M1 midpoints
    K = 64
    zero = np.zeros((1, 4, K), np.float32)
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(4, K)).astype(np.uint8)
    codes[:, ::16] = 7
    codes[codes == 8] = 0
    grid = (F.e2m1_decode(codes) * 448.0).astype(np.float32)[None]
    tiny = (rng.standard_normal((1, 4, K)) * 1e-3).astype(np.float32)
    tiny[0, :, :16] *= 1e-5                    # blocks far below the tensor max
    mids = np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2, np.float32), (4, K // 16))
    mids = (mids * 448.0 * np.sign(rng.standard_normal((4, K)))).astype(np.float32)[None]
    for arr in (zero, grid, tiny, mids):
        bits = S.f32_to_bf16_bits(arr)
        out = moe.Nvfp4Weights.empty(1, 4, K)
        moe.nvfp4_quantize(_bits(bits), out)
        torch.cuda.synchronize()
        p, s, g = quantize(F.bf16_bits_to_f64(bits[0]))
        assert np.array_equal(out.packed.cpu().numpy()[0], p)
        assert np.array_equal(out.scales.cpu().numpy()[0], s)
        assert float(out.global_scale.cpu().numpy()[0]) == g


# ------------------------------------------------------------------- decode
def _tiled_reference(packed, scales):
    """numpy statement of the tiled layout (header: MOE_LAYOUT_TILED)."""
    E, N, K2 = packed.shape
    K = 2 * K2
    tp = np.zeros_like(packed).reshape(E, -1)
    ts = np.zeros_like(scales).reshape(E, -1)
    for n in range(N):
        t, r = divmod(n, 16)
        for k in range(0, K, 32):
            u, g = divmod(k, 128)
            g //= 32
            lane = 16 * g + r
            o = t * 16 * (K // 2) + u * 1024 + lane * 16
            tp[:, o:o + 16] = packed[:, n, k // 2:k // 2 + 16]
            so = t * K + u * 128 + lane * 2
            ts[:, so:so + 2] = scales[:, n, k // 16:k // 16 + 2]
    return tp.reshape(packed.shape), ts.reshape(scales.shape)


@pytest.mark.parametrize("N,K", [(16, 96), (48, 704), (32, 2816)])
def test_repack_matches_layout_definition(N, K):
    rng = np.random.default_rng(N + K)
    packed = rng.integers(0, 256, size=(2, N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(2, N, K // 16), dtype=np.uint8)
    w = moe.Nvfp4Weights(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(),
                         torch.ones(2, dtype=torch.float32, device="cuda"))
    t = moe.nvfp4_repack(w)
    torch.cuda.synchronize()
    rp, rs = _tiled_reference(packed, scales)
    assert np.array_equal(t.packed.cpu().numpy(), rp)
    assert np.array_equal(t.scales.cpu().numpy(), rs)


@pytest.mark.parametrize("N,K", [(32, 64), (704, 2816), (2816, 704)])
@pytest.mark.parametrize("tiled", [False, True])
def test_dequant_bf16_bit_exact(N, K, tiled):
    rng = np.random.default_rng(K)
    E = 2
    packed = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(E, N, K // 16), dtype=np.uint8)  # every finite >= 0 code
    scales[0, 0, :] = np.arange(K // 16) % 0x7F
    w = moe.Nvfp4Weights(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(),
                         torch.ones(E, dtype=torch.float32, device="cuda"))
    if tiled:
        w = moe.nvfp4_repack(w)
    out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        moe.nvfp4_dequant_bf16(w, e, out)
        torch.cuda.synchronize()
        ref = F.dequantize_no_global(packed[e], scales[e])
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref)


def test_dequant_every_scale_code_and_element():
    # all 127 finite non-negative scale codes x all 16 element codes
    K = 16 * 128
    codes = np.tile(np.arange(16, dtype=np.uint8), 128)[None, :]
    packed = F.pack_nibbles(codes)[None]
    scales = np.concatenate([np.arange(0x7F), [0x38]]).astype(np.uint8)[None, None, :]
    w = moe.Nvfp4Weights(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(),
                         torch.ones(1, dtype=torch.float32, device="cuda"))
    out = torch.empty((1, K), dtype=torch.bfloat16, device="cuda")
    moe.nvfp4_dequant_bf16(w, 0, out)
    torch.cuda.synchronize()
    ref = F.dequantize_no_global(packed[0], scales[0])
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), ref)


# ------------------------------------------------------------------- router
def _route_gpu(x_bits, p, k, E):
    T = x_bits.shape[0]
    wr, sc, pes, bias = W.router_to_device(p)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    wr_raw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.moe_route(_bits(x_bits), wr, sc, pes, bias, k, 1e-6, idx, w, wr_raw, lg)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), wr_raw.cpu().numpy(), lg.cpu().numpy()


@pytest.mark.parametrize("T,zipf,outliers", [(1, False, False), (4, False, False), (8192, True, True),
                                             (64, False, False), (333, True, False),
                                             (2048, True, True)])
def test_route_model_shape(T, zipf, outliers):
    p = S.router_params(0, zipf=zipf)
    x = S.activations(90, T, outliers=outliers)
    idx, w, w_raw, lg = _route_gpu(x, p, 8, 128)
    r = router_f64(p)
    ref = M.route(F.bf16_bits_to_f64(x), r["w_router"], r["scale"], r["per_expert_scale"], 8,
                  r["bias"])
    assert np.max(np.abs(lg - ref["logits"])) <= 2e-7
    differ = check_route(idx, w, w_raw, ref, r["per_expert_scale"])
    assert len(differ) <= max(1, T // 200)


@pytest.mark.parametrize("T,E,k,H,zipf", [(1, 128, 8, 2816, False), (37, 128, 8, 2816, False),
                                          (64, 128, 8, 2816, False), (2048, 128, 8, 2816, True),
                                          (130, 256, 16, 2816, False), (9, 64, 4, 192, False),
                                          (70, 32, 3, 4160, True)])
def test_route_without_logits_buffer(T, E, k, H, zipf):
    """moe_route with logits NULL (logits kept in LDS, selection in the same
    kernel): the routing bar against the oracle, and the same ids and
    weights as the call with a logits buffer outside near-ties."""
    router = S.router_params(3, h=H, e=E, zipf=zipf)
    x = S.activations(95, T, h=H)
    wr, sc, pes, bias = W.router_to_device(router)
    outs = []
    for with_logits in (False, True):
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        wraw = torch.empty((T, k), dtype=torch.float32, device="cuda")
        lg = torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None
        moe.moe_route(_bits(x), wr, sc, pes, bias, k, 1e-6, idx, w, wraw, lg)
        torch.cuda.synchronize()
        outs.append((idx.cpu().numpy(), w.cpu().numpy(), wraw.cpu().numpy()))
    r = router_f64(router)
    ref = M.route(F.bf16_bits_to_f64(x), r["w_router"], r["scale"], r["per_expert_scale"], k,
                  r["bias"])
    idx0, w0, wr0 = outs[0]
    check_route(idx0, w0, wr0, ref, r["per_expert_scale"])
    same = np.array([set(a) == set(b) for a, b in zip(idx0.tolist(), outs[1][0].tolist())])
    assert np.all(same | ref["near_tie"])


def test_route_small_odd_shapes():
    for (t, h, e, k) in [(1, 64, 16, 1), (3, 192, 16, 2), (5, 64, 32, 4), (7, 2816, 256, 16),
                         (65, 128, 32, 4), (100, 2816, 256, 8)]:
        c = S.small_case(t + e, t, h, 64, e, k, zipf=(t == 5))
        idx, w, w_raw, lg = _route_gpu(c["x"], c["router"], k, e)
        r = router_f64(c["router"])
        ref = M.route(F.bf16_bits_to_f64(c["x"]), r["w_router"], r["scale"], r["per_expert_scale"],
                      k, r["bias"])
        assert np.max(np.abs(lg - ref["logits"])) <= 2e-7
        check_route(idx, w, w_raw, ref, r["per_expert_scale"])


def test_route_zero_row_and_ties():
    # a zero row has all-zero logits: every expert ties, the lowest ids win
    p = S.router_params(0)
    x = np.zeros((2, 2816), np.uint16)
    x[1] = S.activations(91, 1)[0]
    idx, w, w_raw, lg = _route_gpu(x, p, 8, 128)
    assert sorted(idx[0].tolist()) == list(range(8))
    assert np.allclose(w_raw[0], 1 / 8, atol=1e-7)


# ------------------------------------------------------------------- bucket
def _bucket_gpu(idx, E):
    T, k = idx.shape
    ti = torch.from_numpy(idx.astype(np.int32)).cuda()
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pr = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_bucket_workspace_bytes(T, k, E), dtype=torch.uint8, device="cuda")
    moe.moe_bucket(ti, E, off, sp, pr, ws)
    torch.cuda.synchronize()
    return off.cpu().numpy(), sp.cpu().numpy(), pr.cpu().numpy(), int(ws[:4].view(torch.int32)[0])


@pytest.mark.parametrize("T,k,E,skew", [(0, 8, 128, 0), (1, 8, 128, 0), (4, 8, 128, 0), (64, 8, 128, 0),
                                        (511, 8, 128, 0), (513, 8, 128, 1), (2048, 8, 128, 1),
                                        (16384, 8, 128, 1), (37, 3, 5, 0), (100, 16, 256, 0)])
def test_bucket_bit_exact(T, k, E, skew):
    rng = np.random.default_rng(T * 31 + k)
    if skew:
        pr = 1.0 / np.arange(1, E + 1) ** 1.2
        pr /= pr.sum()
        idx = np.stack([rng.choice(E, k, replace=False, p=pr) for _ in range(T)]) if T else np.zeros((0, k), int)
    else:
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]) if T else np.zeros((0, k), int)
    off, sp, pr_, err = _bucket_gpu(idx, E)
    ref = M.bucket(idx, E)
    assert err == 0
    assert np.array_equal(off, ref["offsets"])
    assert np.array_equal(sp, ref["sorted_pairs"])
    assert np.array_equal(pr_, ref["pair_rank"])


@pytest.mark.parametrize("T", [5, 700])
def test_bucket_invalid_ids_counted_and_parked(T):
    k, E = 4, 16
    rng = np.random.default_rng(T)
    idx = rng.integers(0, E, size=(T, k))
    bad = rng.random((T, k)) < 0.1
    idx[bad] = np.where(rng.random(bad.sum()) < 0.5, -3, E + 7)
    off, sp, pr, err = _bucket_gpu(idx, E)
    assert err == int(bad.sum())
    flat = idx.reshape(-1)
    key = [(int(e) if 0 <= e < E else E, p) for p, e in enumerate(flat)]
    order = [p for _, p in sorted(key)]
    assert np.array_equal(sp, np.array(order))
    valid = ~bad.reshape(-1)
    assert np.array_equal(sp[pr[valid]], np.arange(T * k)[valid])
    assert np.all(pr[~valid] == -1)                  # no rank: the combine skips them
    assert off[E] == T * k - err


def test_invalid_ids_contribute_nothing_through_the_combine():
    """Pairs whose expert id is out of range are counted, get rank -1 and add
    nothing: bucket -> expert MLP -> combine equals the oracle block on the
    valid pairs only (their routing weights left as given)."""
    T, k, E, H, I = 9, 4, 16, 128, 64
    c = S.small_case(61, T, H, I, E, k)
    layer = W.build_small_layer(c, k)
    rng = np.random.default_rng(61)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    bad = np.zeros((T, k), bool)
    bad[[0, 3, 3, 8], [1, 0, 2, 3]] = True
    idx_bad = idx.copy()
    idx_bad[bad] = np.array([-1, E, E + 5, -7])
    off, sp, pr, err = _bucket_gpu(idx_bad, E)
    assert err == int(bad.sum())
    assert np.all(pr.reshape(T, k)[bad] == -1) and np.all(pr.reshape(T, k)[~bad] >= 0)
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    moe.nvfp4_expert_mlp(_bits(c["x"]), layer.gate, layer.up, layer.down,
                         torch.from_numpy(off).cuda(), torch.from_numpy(sp).cuda(), k, y, ws)
    w = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(y, torch.from_numpy(w).cuda(), torch.from_numpy(pr).cuda(), out)
    torch.cuda.synchronize()
    q = {n: quantize_experts(F.bf16_bits_to_f64(c[n])) for n in ("gate", "up", "down")}
    fns = {n: M.nvfp4_weights(*q[n]) for n in q}
    xs = F.bf16_bits_to_f64(c["x"])
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if not bad[t, j]:
                e = int(idx[t, j])
                ref[t] += w[t, j] * M.expert_mlp(xs[t:t + 1], fns["gate"](e), fns["up"](e),
                                                 fns["down"](e))[0]
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert rel_frob(got, ref) <= REL_FROB_TOL


# ---------------------------------------------- fused routing + bucketing
@pytest.mark.parametrize("T,H,E,k", [(0, 2816, 128, 8), (1, 2816, 128, 8), (4, 2816, 128, 8), (16, 2816, 128, 8), (33, 2816, 128, 8), (64, 2816, 256, 16),
                                     (17, 2816, 128, 8), (64, 2816, 128, 8), (65, 2816, 128, 8),
                                     (333, 2816, 128, 8), (9, 192, 16, 3), (64, 4096, 256, 16),
                                     (30, 4160, 32, 4)])
def test_route_bucket_matches_oracle_and_separate_calls(T, H, E, k):
    """moe_route_bucket: the routing against the oracle (the same bar as
    moe_route), the bucketing bit-exact against the oracle's bucketing of the
    experts it chose, and for T <= 64 every output byte equal to moe_route +
    moe_bucket (more tokens take the K-split logits: moe_route's ids outside
    near-ties, and the bucketing equal to moe_bucket of its own ids)."""
    router = S.router_params(E % 7, h=H, e=E, zipf=(T == 17))
    x = S.activations(93, T, h=H)
    wr, sc, pes, bias = W.router_to_device(router)
    xd = _bits(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    wsb = moe.moe_bucket_workspace_bytes(T, k, E)

    def outs():
        return dict(idx=torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
                    w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
                    w_raw=torch.empty((T, k), dtype=torch.float32, device="cuda"),
                    lg=torch.empty((T, E), dtype=torch.float32, device="cuda"),
                    off=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
                    sp=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
                    pr=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
                    ws=torch.full((wsb,), 0x55, dtype=torch.uint8, device="cuda"))
    a, b = outs(), outs()
    moe.moe_route_bucket(xd, wr, sc, pes, bias, k, 1e-6, a["idx"], a["w"], a["w_raw"], a["lg"],
                         a["off"], a["sp"], a["pr"], a["ws"])
    moe.moe_route(xd, wr, sc, pes, bias, k, 1e-6, b["idx"], b["w"], b["w_raw"], b["lg"])
    split = T > 64
    if split:
        b_idx = b["idx"].clone()
        b["idx"].copy_(a["idx"])
    moe.moe_bucket(b["idx"], E, b["off"], b["sp"], b["pr"], b["ws"])
    torch.cuda.synchronize()
    for n in ("off", "sp", "pr") if split else ("idx", "w", "w_raw", "lg", "off", "sp", "pr"):
        assert torch.equal(a[n].view(torch.int32), b[n].view(torch.int32)), n
    assert int(a["ws"][:4].view(torch.int32)[0]) == 0
    idx = a["idx"].cpu().numpy()
    ref_b = M.bucket(idx, E)
    assert np.array_equal(a["off"].cpu().numpy(), ref_b["offsets"])
    assert np.array_equal(a["sp"].cpu().numpy(), ref_b["sorted_pairs"])
    assert np.array_equal(a["pr"].cpu().numpy(), ref_b["pair_rank"])
    if T:
        r = router_f64(router)
        ref = M.route(F.bf16_bits_to_f64(x), r["w_router"], r["scale"], r["per_expert_scale"], k,
                      r["bias"])
        assert np.max(np.abs(a["lg"].cpu().numpy() - ref["logits"])) <= 2e-7
        differ = check_route(idx, a["w"].cpu().numpy(), a["w_raw"].cpu().numpy(), ref,
                             r["per_expert_scale"])
        assert len(differ) <= max(1, T // 200)
        if split:
            same = np.array([set(u) == set(v) for u, v in zip(idx.tolist(), b_idx.cpu().numpy().tolist())])
            assert np.all(same | ref["near_tie"])


@pytest.mark.parametrize("T,H,E,k", [(65, 2816, 128, 8), (2048, 2816, 128, 8), (4096, 2816, 128, 8),
                                     (16384, 2816, 128, 8), (700, 4160, 32, 4), (5000, 192, 16, 3),
                                     (300, 2816, 256, 16)])
def test_route_bucket_split_logits(T, H, E, k):
    """The K-split router logits of moe_route_bucket (up to 8 slices of H,
    64 x 32 or 64 x 128 tiles; H = 4160 ends in half a chunk, H = 192 has
    two chunks for more slices asked, E = 256 selects from 4 experts per
    lane): logits within 2e-7 of the oracle with and without a logits buffer,
    the ids and weights against the oracle, and equal results whether or
    not the logits are written out."""
    router = S.router_params(T % 5, h=H, e=E, zipf=(T == 2048 or T == 16384))
    x = S.activations(97, T, h=H, outliers=(T == 16384))
    wr, sc, pes, bias = W.router_to_device(router)
    wsb = moe.moe_bucket_workspace_bytes(T, k, E)
    res = []
    for with_logits in (True, False):
        o = dict(idx=torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
                 w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
                 w_raw=torch.empty((T, k), dtype=torch.float32, device="cuda"),
                 lg=torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None,
                 off=torch.empty((E + 1,), dtype=torch.int32, device="cuda"),
                 sp=torch.empty((T * k,), dtype=torch.int32, device="cuda"),
                 pr=torch.empty((T * k,), dtype=torch.int32, device="cuda"),
                 ws=torch.full((wsb,), 0x55, dtype=torch.uint8, device="cuda"))
        moe.moe_route_bucket(_bits(x), wr, sc, pes, bias, k, 1e-6, o["idx"], o["w"], o["w_raw"],
                             o["lg"], o["off"], o["sp"], o["pr"], o["ws"])
        torch.cuda.synchronize()
        res.append(o)
    for n in ("idx", "w", "w_raw", "off", "sp", "pr"):
        assert torch.equal(res[0][n], res[1][n]), n
    r = router_f64(router)
    ref = M.route(F.bf16_bits_to_f64(x), r["w_router"], r["scale"], r["per_expert_scale"], k,
                  r["bias"])
    assert np.max(np.abs(res[0]["lg"].cpu().numpy() - ref["logits"])) <= 2e-7
    idx = res[0]["idx"].cpu().numpy()
    differ = check_route(idx, res[0]["w"].cpu().numpy(), res[0]["w_raw"].cpu().numpy(), ref,
                         r["per_expert_scale"])
    assert len(differ) <= max(1, T // 200)
    ref_b = M.bucket(idx, E)
    assert np.array_equal(res[0]["off"].cpu().numpy(), ref_b["offsets"])
    assert np.array_equal(res[0]["sp"].cpu().numpy(), ref_b["sorted_pairs"])


@pytest.mark.parametrize("T,H,E,k,I", [(0, 2816, 128, 8, 704), (1, 2816, 128, 8, 704),
                                       (5, 2816, 128, 8, 704), (64, 2816, 128, 8, 704),
                                       (65, 2816, 128, 8, 704), (300, 2816, 128, 8, 704),
                                       (1024, 2816, 128, 8, 704), (1100, 4160, 32, 4, 64),
                                       (9, 192, 16, 3, 64), (64, 4096, 256, 16, 128),
                                       (30, 4160, 32, 4, 64)])
@pytest.mark.parametrize("norm", [False, True])
def test_route_bucket_prep_equals_separate_calls(T, H, E, k, I, norm):
    """moe_route_bucket_prep: every output byte, the whole expert workspace
    included (filled with garbage first, so that the clearing of the row
    maxima is checked), equal to moe_route_bucket followed by
    nvfp4_expert_prep (or nvfp4_expert_prep_rmsnorm); T = 1024 and 1100 have
    more than 4096 pairs (the chunked bucketing), and H = 4160 rows are
    longer than a wave of the prep keeps in registers."""
    router = S.router_params(3, h=H, e=E)
    x = S.activations(94, T, h=H)
    x[:min(T, 2)] = S.f32_to_bf16_bits(S.bf16_bits_to_f32(x[:min(T, 2)]) * np.float32(3e4))
    wr, sc, pes, bias = W.router_to_device(router)
    xd = _bits(x) if T else torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    nw = _bits(S.norm_weights(2, h=H)[0]) if norm else None
    wsb = moe.moe_bucket_workspace_bytes(T, k, E)
    wse = moe.moe_workspace_bytes(T, k, E, H, I)

    def outs():
        return dict(idx=torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
                    w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
                    w_raw=torch.empty((T, k), dtype=torch.float32, device="cuda"),
                    lg=torch.empty((T, E), dtype=torch.float32, device="cuda"),
                    off=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
                    sp=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
                    pr=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
                    ws=torch.full((wsb,), 0x55, dtype=torch.uint8, device="cuda"),
                    ews=torch.full((wse,), 0xA7, dtype=torch.uint8, device="cuda"))
    a, b = outs(), outs()
    moe.moe_route_bucket_prep(xd, wr, sc, pes, bias, k, 1e-6, a["idx"], a["w"], a["w_raw"],
                              a["lg"], a["off"], a["sp"], a["pr"], a["ws"], nw, 1e-6, I, a["ews"])
    moe.moe_route_bucket(xd, wr, sc, pes, bias, k, 1e-6, b["idx"], b["w"], b["w_raw"], b["lg"],
                         b["off"], b["sp"], b["pr"], b["ws"])
    if norm:
        moe.nvfp4_expert_prep_rmsnorm(xd, nw, 1e-6, E, I, k, b["ews"])
    else:
        moe.nvfp4_expert_prep(xd, E, I, k, b["ews"])
    torch.cuda.synchronize()
    for n in ("idx", "w", "w_raw", "lg", "off", "sp", "pr", "ews"):
        assert torch.equal(a[n].view(torch.uint8), b[n].view(torch.uint8)), n
    assert int(a["ws"][:4].view(torch.int32)[0]) == 0


# ---------------------------------------------------------------- experts
def _expert_case(T, k, E, H, I, seed):
    c = S.small_case(seed, T, H, I, E, k)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    return c, idx


# Shapes chosen to reach every kernel variant: GEMV mode with 8-row tiles
# (1 and 2 row groups, experts split over several tiles), GEMV mode with
# 16-row tiles (1 to 4 row groups), and the LDS-tiled GEMM with 32- and
# 64-row tiles; odd H / I multiples of 64 leave partial K units; H = 4160
# takes the prep path for rows longer than the registers keep.
@pytest.mark.parametrize("T,k,E,H,I", [(1, 2, 8, 128, 64), (5, 2, 8, 128, 64), (16, 2, 8, 128, 64),
                                       (24, 4, 16, 256, 128), (37, 4, 8, 192, 128),
                                       (100, 4, 8, 128, 64), (300, 2, 4, 256, 64),
                                       (100, 4, 8, 192, 128), (200, 2, 4, 64, 64),
                                       (3, 1, 2, 4160, 64)])
def test_expert_mlp_small(T, k, E, H, I):
    c, idx = _expert_case(T, k, E, H, I, seed=T)
    _check_expert_mlp(c, idx, T, k, E, H, I)


def test_expert_mlp_skewed_gemv_mode():
    # GEMV mode (fewer than 24 rows per active expert on average) with popular
    # experts far above one tile of rows (several tiles each) next to experts
    # with a handful of rows
    T, k, E, H, I = 300, 8, 128, 128, 64
    c = S.small_case(123, T, H, I, E, k)
    rng = np.random.default_rng(5)
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    p /= p.sum()
    idx = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    counts = np.bincount(idx.ravel(), minlength=E)
    assert counts.max() > 64 and 0 < (counts[counts > 0] <= 32).sum() and T * k < 24 * E
    _check_expert_mlp(c, idx, T, k, E, H, I)


def test_expert_mlp_gemm_every_row_group():
    # LDS-tiled GEMM mode (64-row blocks) with bucket sizes chosen so that
    # blocks hold 1..16, 17..32, 33..48 and 49..64 rows (each count of 16-row
    # groups the kernels specialise on), full and ragged, an expert of 10 row
    # blocks (block groups of 8 with a shorter last group) and empty experts;
    # H = 192 leaves half a K unit and down waves past N, I = 64 leaves gate/up
    # waves past N
    sizes = [1, 16, 17, 33, 48, 49, 64, 130, 600]
    k, E, H, I = 1, 16, 192, 64
    T = sum(sizes)
    c = S.small_case(2024, T, H, I, E, k)
    rng = np.random.default_rng(11)
    experts = rng.permutation(E)[:len(sizes)]
    idx = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in zip(experts, sizes)])
    idx = idx[rng.permutation(T)].reshape(T, k)
    assert sorted(np.bincount(idx.ravel(), minlength=E)[experts]) == sorted(sizes)
    _check_expert_mlp(c, idx, T, k, E, H, I)


def test_expert_mlp_gemm_128_row_blocks():
    # buckets of 128 rows or more on average take the expert GEMMs with
    # 128-row blocks (accumulators in the accumulation registers): bucket
    # sizes whose last block holds 1, 17..32, 33..64 and 65..128 rows (each
    # count of 16-row groups that kernel specialises on), a full block, and
    # experts of 3, 6 and 14 blocks (block groups of 8 with a shorter last
    # group); H = 192 leaves half a K unit, I = 64 leaves waves past N
    sizes = [1, 20, 50, 100, 128, 300, 700, 1773]
    k, E, H, I = 1, 8, 192, 64
    T = sum(sizes)
    assert T * k // min(T * k, E) >= 128
    c = S.small_case(2025, T, H, I, E, k)
    rng = np.random.default_rng(12)
    experts = rng.permutation(E)[:len(sizes)]
    idx = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in zip(experts, sizes)])
    idx = idx[rng.permutation(T)].reshape(T, k)
    assert sorted(np.bincount(idx.ravel(), minlength=E)[experts]) == sorted(sizes)
    _check_expert_mlp(c, idx, T, k, E, H, I)


@pytest.mark.parametrize("E,sizes", [
    # 128-row blocks: one expert of 12 blocks beside tails of 1..129 rows and empty experts
    (16, [1500, 600, 300, 129, 64, 40, 17, 16, 5, 1]),
    # 64-row blocks: the same skew over more experts, most of them small
    (64, [900, 300, 65, 48, 33, 20, 17, 9, 3, 2, 1, 1, 1] + [4] * 30),
])
def test_expert_mlp_gemm_cost_balanced_split(E, sizes):
    # the gate/up blocks are spread over the XCDs in ranges of equal cost
    # (not equal counts): skewed buckets with empty experts, where the ranges
    # differ most from the count split and some reach their length cap
    k, H, I = 1, 192, 64
    T = sum(sizes)
    c = S.small_case(2026 + E, T, H, I, E, k)
    rng = np.random.default_rng(E)
    experts = rng.permutation(E)[:len(sizes)]
    idx = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in zip(experts, sizes)])
    idx = idx[rng.permutation(T)].reshape(T, k)
    _check_expert_mlp(c, idx, T, k, E, H, I)


def _check_expert_mlp(c, idx, T, k, E, H, I):
    layer = W.build_small_layer(c, k)
    off, sp, pr, _ = _bucket_gpu(idx, E)
    x = _bits(c["x"])
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    moe.nvfp4_expert_mlp(x, layer.gate, layer.up, layer.down, torch.from_numpy(off).cuda(),
                         torch.from_numpy(sp).cuda(), k, y, ws)
    torch.cuda.synchronize()
    q = {n: quantize_experts(F.bf16_bits_to_f64(c[n])) for n in ("gate", "up", "down")}
    fns = {n: M.nvfp4_weights(*q[n]) for n in q}
    ref = M.experts(F.bf16_bits_to_f64(c["x"]), M.bucket(idx, E), k, fns["gate"], fns["up"], fns["down"])
    got = y.float().cpu().numpy()
    assert rel_frob(got, ref) <= 5e-3
    assert np.max(row_rel(got, ref)) <= 1e-2


def test_expert_mlp_large_activation_rows():
    # rows spanning a wide range (1e-17 .. 1e15 in one batch; the intermediate
    # A then spans about 1e-36 .. 1e30, inside the bf16 range) stay finite and
    # accurate thanks to the per-row power-of-two rescale; the 1e-17 row's A
    # (below 2^-110) takes the clamped exponent, whose factor 2^124 is finite
    # (unclamped it would be 2^131: inf).  A 1e-19 row makes A subnormal in
    # bf16: that row only has to stay finite.
    T, k, E, H, I = 7, 2, 4, 128, 64
    c, idx = _expert_case(T, k, E, H, I, seed=77)
    xf = S.bf16_bits_to_f32(c["x"]).copy()
    xf[1] *= 1e15
    xf[2] *= 1e-15
    xf[3] *= 3e4
    xf[4] *= 1e-17
    xf[6] *= 1e-19
    c["x"] = S.f32_to_bf16_bits(xf)
    layer = W.build_small_layer(c, k)
    off, sp, pr, _ = _bucket_gpu(idx, E)
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    moe.nvfp4_expert_mlp(_bits(c["x"]), layer.gate, layer.up, layer.down,
                         torch.from_numpy(off).cuda(), torch.from_numpy(sp).cuda(), k, y, ws)
    torch.cuda.synchronize()
    q = {n: quantize_experts(F.bf16_bits_to_f64(c[n])) for n in ("gate", "up", "down")}
    fns = {n: M.nvfp4_weights(*q[n]) for n in q}
    ref = M.experts(F.bf16_bits_to_f64(c["x"]), M.bucket(idx, E), k, fns["gate"], fns["up"], fns["down"])
    got = y.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    tok = np.asarray(M.bucket(idx, E)["sorted_pairs"]) // k     # token of each sorted row
    assert np.max(row_rel(got[tok != 6], ref[tok != 6])) <= 1e-2   # all but the 1e-19 token
    assert float(np.max(np.abs(ref[tok == 4]))) < 1e-30          # the 1e-17 token is that small


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("T,k,H", [(1, 8, 2816), (9, 3, 64), (64, 8, 2816)])
def test_combine(T, k, H):
    rng = np.random.default_rng(T + k)
    P = T * k
    y = S.f32_to_bf16_bits(rng.standard_normal((P, H)).astype(np.float32))
    w = rng.uniform(0.05, 1.5, (T, k)).astype(np.float32)
    rank = rng.permutation(P).astype(np.int32)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(_bits(y), torch.from_numpy(w).cuda(), torch.from_numpy(rank).cuda(), out)
    torch.cuda.synchronize()
    ref = M.combine(F.bf16_bits_to_f64(y), w.astype(np.float64), rank, k)
    got = out.float().cpu().numpy()
    # one bf16 rounding of an fp32 sum: |err| <= 2^-8 |ref| + fp32 slack
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())


# ------------------------------------------------ combine + the layer step's norms
@pytest.mark.parametrize("T,k,H,mode,alias", [(5, 3, 2816, "step_h1", None), (7, 8, 200, "branch", None),
                                              (3, 8, 8192, "step", "residual"),
                                              (64, 8, 2816, "step_h1", None),
                                              (2, 16, 64, "step_h1", "h1"),
                                              (4, 8, 2816, "step_h1", "residual")])
def test_combine_rmsnorm(T, k, H, mode, alias):
    """h2 = rmsnorm(sum_j w_j y_j, w2); the layer step (residual +
    rmsnorm(h1 + h2, w)) * scalar, or h2 alone ("Gemma 4 26B-A4B (MoE) - Core
    AI", Architecture code sketch), against the oracle's norms in fp64."""
    rng = np.random.default_rng(100 * T + k)
    P = T * k
    y = S.f32_to_bf16_bits(rng.standard_normal((P, H)).astype(np.float32))
    w = rng.uniform(0.05, 1.5, (T, k)).astype(np.float32)
    rank = rng.permutation(P).astype(np.int32)
    g2 = S.f32_to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    g = S.f32_to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32))
    res = S.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    h1 = S.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    scalar = 0.625
    step = mode != "branch"
    res_d = _bits(res) if step else None
    h1_d = _bits(h1) if mode == "step_h1" else None
    out = {"residual": res_d, "h1": h1_d}.get(alias)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_rmsnorm(_bits(y), torch.from_numpy(w).cuda(), torch.from_numpy(rank).cuda(),
                            _bits(g2), 1e-6, out, h1=h1_d, post_norm=_bits(g) if step else None,
                            residual=res_d, layer_scalar=scalar)
    torch.cuda.synchronize()
    s_ = M.combine(F.bf16_bits_to_f64(y), w.astype(np.float64), rank, k)
    ref = M.rms_norm(s_, F.bf16_bits_to_f64(g2), 1e-6)
    if step:
        u = ref + (F.bf16_bits_to_f64(h1) if mode == "step_h1" else 0.0)
        ref = (F.bf16_bits_to_f64(res) + M.rms_norm(u, F.bf16_bits_to_f64(g), 1e-6)) * scalar
    got = out.float().cpu().numpy()
    # fp32 sums, norms and residual add, one bf16 rounding
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())


def test_combine_rmsnorm_empty_batch():
    out = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_rmsnorm(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                            torch.empty((0, 8), dtype=torch.float32, device="cuda"),
                            torch.empty((0,), dtype=torch.int32, device="cuda"), g, 1e-6, out)
    torch.cuda.synchronize()
