"""GPU parity of the int4 expert formats ("Gemma 4 26B-A4B (MoE) - Core AI",
Compression recipe: q4_0, w = (q - 8) d, and affine aff4, w = q s + b, one
fp16 scale (and bias) per 32 weights) on the same expert kernels as NVFP4:
the tiled repack against the layout's definition, the kernels' weight decode
bit-exact against the oracle's exact value rounded once to f16, and the expert
MLP and the whole block against the fp64 oracle."""
import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import formats as F
from oracle import int4 as Q
from oracle import moe as M

import nvfp4_weight_only_moe_amd as moe
from nvfp4_weight_only_moe_amd import workload as W

from parity_util import REL_FROB_TOL, check_route, rel_frob, router_f64, row_rel

pytestmark = pytest.mark.gpu

FMTS = ("q4_0", "aff4")


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available()
    moe.lib()


def _sbits(fmt, scale_bytes):
    """Scale bytes [..., N, K/32 * SB] -> the oracle's fp16 bit arrays."""
    b = np.ascontiguousarray(scale_bytes).view(np.uint16)
    return b if fmt == "q4_0" else b.reshape(b.shape[:-1] + (-1, 2))


def _decode(fmt, packed, scale_bytes):
    dec = Q.decode_q4_0 if fmt == "q4_0" else Q.decode_aff4
    return dec(packed, _sbits(fmt, scale_bytes))


def _oracle_fns(fmt, stacks):
    return {n: (lambda e, n=n: _decode(fmt, stacks[n][0][e], stacks[n][1][e])) for n in stacks}


# -------------------------------------------------------------- tiled layout
def _tiled_int4_reference(packed, scales, sb):
    """numpy statement of the tiled int4 layout (header: nvfp4_tensor): the
    NVFP4 tile order of the packed bytes, the 8 nibbles of each dword
    reordered (byte b <- element b in the low nibble, element b + 4 in the
    high one), and the scales of lane l of unit u of tile t at
    t*K*SB/2 + 64*SB*u + SB*l."""
    E, N, K2 = packed.shape
    K = 2 * K2
    codes = np.empty((E, N, K), dtype=np.uint8)
    codes[..., 0::2] = packed & 15
    codes[..., 1::2] = packed >> 4
    c8 = codes.reshape(E, N, K // 8, 8)
    rebyte = (c8[..., 0:4] | (c8[..., 4:8] << 4)).astype(np.uint8).reshape(E, N, K // 2)
    tp = np.zeros_like(packed).reshape(E, -1)
    ts = np.zeros_like(scales).reshape(E, -1)
    for n in range(N):
        t, r = divmod(n, 16)
        for k in range(0, K, 32):
            u, g = divmod(k, 128)
            g //= 32
            lane = 16 * g + r
            o = t * 16 * (K // 2) + u * 1024 + lane * 16
            tp[:, o:o + 16] = rebyte[:, n, k // 2:k // 2 + 16]
            so = t * K * sb // 2 + u * 64 * sb + lane * sb
            ts[:, so:so + sb] = scales[:, n, (k // 32) * sb:(k // 32 + 1) * sb]
    return tp.reshape(packed.shape), ts.reshape(scales.shape)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(16, 96), (48, 704), (32, 2816)])
def test_int4_repack_matches_layout_definition(fmt, N, K):
    rng = np.random.default_rng(N + K)
    sb = S.INT4_SCALE_BYTES[fmt]
    packed = rng.integers(0, 256, size=(2, N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(2, N, K // 32 * sb), dtype=np.uint8)
    t = moe.nvfp4_repack(W.int4_to_device(fmt, packed, scales, tiled=False))
    torch.cuda.synchronize()
    assert t.format == moe.FORMATS[fmt] and t.layout == moe.LAYOUT_TILED
    rp, rs = _tiled_int4_reference(packed, scales, sb)
    assert np.array_equal(t.packed.cpu().numpy(), rp)
    assert np.array_equal(t.scales.cpu().numpy(), rs)


# ------------------------------------------------------------------ decode
def _edge_scales(fmt, rng, N, K):
    """fp16 scales that reach the corners of the decode: zero, signed zero,
    subnormals, the smallest normal, exact powers of two, values whose
    products round (and, for aff4, overflow to inf), negative scales."""
    nb = K // 32
    special = np.array([0.0, -0.0, 2.0 ** -24, 3 * 2.0 ** -24, 2.0 ** -14, 1.0, -1.0, 0.0999,
                        1023.5, -8188.0, 8188.0, 3.1416, -0.00611, 6.1e-5, 0.5, 2.0],
                       dtype=np.float16)
    if fmt == "q4_0":
        d = rng.uniform(-0.01, 0.01, (N, nb)).astype(np.float16)
        d.flat[:len(special)] = special
        return d.view(np.uint8).reshape(N, -1)
    sb = np.empty((N, nb, 2), dtype=np.float16)
    sb[..., 0] = rng.uniform(-0.01, 0.01, (N, nb))
    sb[..., 1] = rng.uniform(-0.06, 0.06, (N, nb))
    sb[..., 0].flat[:len(special)] = special
    sb[..., 1].flat[:len(special)] = special[::-1]
    sb[0, -1] = (np.float16(60000.0), np.float16(30000.0))     # q s + b overflows to inf
    sb[1, -1] = (np.float16(-60000.0), np.float16(-30000.0))   # ... and to -inf
    return np.ascontiguousarray(sb).view(np.uint8).reshape(N, -1)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(32, 64), (704, 2816), (2816, 704)])
@pytest.mark.parametrize("tiled", [False, True])
def test_int4_dequant_f16_bit_exact(fmt, N, K, tiled):
    rng = np.random.default_rng(K + (fmt == "aff4"))
    E = 2
    packed = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    # every code in both nibble positions within the first 32 weights of row 0
    packed[0, 0, :16] = [(i << 4) | (15 - i) for i in range(16)]
    scales = np.stack([_edge_scales(fmt, rng, N, K) for _ in range(E)])
    w = W.int4_to_device(fmt, packed, scales, tiled=tiled)
    out = torch.empty((N, K), dtype=torch.float16, device="cuda")
    for e in range(E):
        moe.moe_dequant_f16(w, e, out)
        torch.cuda.synchronize()
        ref = Q.round_f16(_decode(fmt, packed[e], scales[e]))
        got = out.cpu().numpy().astype(np.float64)
        # values compare exactly (a zero weight may come out as +0 where the
        # exact product is -0: the sign of a zero weight changes no sum)
        assert np.array_equal(got, ref), f"{int(np.sum(got != ref))} of {got.size} differ"


@pytest.mark.parametrize("N,K", [(32, 64), (704, 2816)])
@pytest.mark.parametrize("tiled", [False, True])
def test_nvfp4_dequant_f16_exact(N, K, tiled):
    # E2M1 x E4M3 is exact in f16 (at most 5 significant bits, 2^-10 .. 2688)
    rng = np.random.default_rng(N)
    packed = rng.integers(0, 256, size=(2, N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(2, N, K // 16), dtype=np.uint8)
    w = moe.Nvfp4Weights(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(),
                         torch.ones(2, dtype=torch.float32, device="cuda"))
    if tiled:
        w = moe.nvfp4_repack(w)
    out = torch.empty((N, K), dtype=torch.float16, device="cuda")
    for e in range(2):
        moe.moe_dequant_f16(w, e, out)
        torch.cuda.synchronize()
        ref = F.dequantize_no_global(packed[e], scales[e])
        assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


# ----------------------------------------------------------------- experts
def _bucket(idx, E):
    T, k = idx.shape
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pr = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_bucket_workspace_bytes(T, k, E), dtype=torch.uint8, device="cuda")
    moe.moe_bucket(torch.from_numpy(idx).cuda(), E, off, sp, pr, ws)
    return off, sp


def _expert_mlp_check(fmt_gu, fmt_d, T, k, E, H, I, seed):
    c = S.small_int4_case(seed, fmt_gu, T, H, I, E, k)
    if fmt_d != fmt_gu:
        c["down"] = S.small_int4_case(seed, fmt_d, T, H, I, E, k)["down"]
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    g, u = (W.int4_to_device(fmt_gu, *c[n]) for n in ("gate", "up"))
    d = W.int4_to_device(fmt_d, *c["down"])
    off, sp = _bucket(idx, E)
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    moe.nvfp4_expert_mlp(W.to_device_bf16(c["x"]), g, u, d, off, sp, k, y, ws)
    torch.cuda.synchronize()
    fg = _oracle_fns(fmt_gu, {n: c[n] for n in ("gate", "up")})
    fd = _oracle_fns(fmt_d, {"down": c["down"]})
    ref = M.experts(F.bf16_bits_to_f64(c["x"]), M.bucket(idx, E), k, fg["gate"], fg["up"],
                    fd["down"])
    got = y.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert rel_frob(got, ref) <= 5e-3
    assert np.max(row_rel(got, ref)) <= 1e-2


# GEMV mode with 8- and 16-row tiles (split and unsplit K) and the GEMM with
# 64- and (T = 1600: 400 rows per expert) 128-row blocks, with
# partial K units (H, I odd multiples of 64)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,k,E,H,I", [(1, 2, 8, 128, 64), (16, 2, 8, 128, 64),
                                       (24, 4, 16, 256, 128), (37, 4, 8, 192, 128),
                                       (300, 2, 4, 256, 64), (100, 4, 8, 192, 128),
                                       (1600, 2, 8, 192, 128)])
def test_int4_expert_mlp_small(fmt, T, k, E, H, I):
    _expert_mlp_check(fmt, fmt, T, k, E, H, I, seed=T + 3)


@pytest.mark.parametrize("T", [5, 300])
def test_mixed_formats_gate_up_and_down(T):
    # q4_0 gate/up with an aff4 down projection (formats are per tensor)
    _expert_mlp_check("q4_0", "aff4", T, 2, 8, 128, 64, seed=11)


# -------------------------------------------------------------- whole block
_LAYERS = {}


def _layer(fmt, zipf):
    key = (fmt, zipf)
    if key not in _LAYERS:
        _LAYERS.clear()   # one model-shaped layer resident at a time
        _LAYERS[key] = W.build_int4_layer(fmt, 0, zipf=zipf)
    return _LAYERS[key]


def _block_check(fmt, zipf, T, sample=None):
    layer = _layer(fmt, zipf)
    x = S.activations(7, T)
    buf = moe.MoeBuffers(T, layer.H, layer.I, layer.E, layer.top_k)
    moe.forward(layer, W.to_device_bf16(x), buf)
    torch.cuda.synchronize()
    rp = S.router_params(0, zipf=zipf)
    r = router_f64(rp)
    xs = F.bf16_bits_to_f64(x)
    toks = np.arange(T) if sample is None else np.asarray(sample)
    ref_r = M.route(xs[toks], r["w_router"], r["scale"], r["per_expert_scale"], 8, r["bias"])
    gidx = buf.topk_idx.cpu().numpy()[toks]
    check_route(gidx, buf.topk_w.cpu().numpy()[toks], buf.topk_w_raw.cpu().numpy()[toks], ref_r,
                r["per_expert_scale"])
    assert buf.bucket_error_count() == 0

    def fn(proj):
        return lambda e: _decode(fmt, *S.int4_expert(fmt, 0, proj, e))
    ref = M.moe_block(xs[toks], xs[toks], r, fn(S.GATE), fn(S.UP), fn(S.DOWN), k=8,
                      ids=gidx.astype(np.int64))["out"]
    got = buf.out.float().cpu().numpy()[toks]
    assert np.all(np.isfinite(got))
    err = rel_frob(got, ref)
    assert err <= REL_FROB_TOL, err
    return err, float(np.max(row_rel(got, ref)))


@pytest.mark.parametrize("fmt", FMTS)
def test_int4_layer_T64_all_tokens(fmt):
    err, worst = _block_check(fmt, False, 64)
    assert worst <= 1e-2
    print(f"{fmt} T=64 rel_frob={err:.3e} worst_row={worst:.3e}")


@pytest.mark.parametrize("fmt", FMTS)
def test_int4_layer_T2048_zipf_sampled(fmt):
    err, _ = _block_check(fmt, True, 2048, np.linspace(0, 2047, 8).astype(int))
    print(f"{fmt} T=2048 zipf rel_frob(sample)={err:.3e}")
