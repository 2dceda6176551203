"""Seeded synthetic inputs for the NVFP4 MoE expert block.

The one source of inputs for both the HIP library and the CPU oracle.  It holds
none of the block's arithmetic: it only draws random numbers, rounds them to
bf16 once, and lays out the workloads.  Shapes are Gemma-4-26B-A4B's ("Gemma 4
26B-A4B (MoE) - Core AI", Architecture table: hidden 2816, 128 experts, top 8,
expert intermediate 704, 30 layers).

Recipe (every value is drawn once and rounded once, round-to-nearest-even):
* seed -> numpy SeedSequence(seed, spawn_key=key) -> PCG64, one stream per key,
  so any single tensor (one expert's projection, one layer's router) can be
  regenerated on its own.
* expert weights: N(0, 0.02) drawn in float32, rounded to bf16; gate and up are
  [I, H] = [704, 2816], down is [H, I] = [2816, 704] per expert.
* router: W [E, H] ~ N(0, H^-0.5); scale [H] ~ U(0.8, 1.2);
  per_expert_scale [E] ~ U(0.5, 1.5); all bf16.
* activations: x [T, H] ~ N(0, 1) bf16; the expert input is the same x.
* skewed routing (prefill workloads): a per-expert logit bias
  b_e = -1.2 * beta * ln(rank_e) with rank a seeded permutation of 1..E and
  beta = sigma_l * sqrt(6) / pi, sigma_l = H^-0.5 * rms(scale), the standard
  deviation of the unbiased logits.  Under the Gumbel-max view of top-k
  selection this makes the first choice roughly Zipf(1.2).
* outlier tokens (long prefill): ceil(0.01 T) rows chosen without replacement
  are multiplied by 20 and rounded to bf16 again.
* int4 expert stacks (the q4_0 and aff4 formats of "Gemma 4 26B-A4B (MoE) -
  Core AI", Compression recipe), drawn directly in the stored form: codes
  uniform on 0..15, two per byte (low nibble = even k); per block of 32 along
  K one fp16 d ~ U(0.004, 0.008) (q4_0), or one fp16 s ~ U(0.004, 0.008) and
  one fp16 b ~ U(-0.06, -0.035) (aff4), rounded to fp16 once.  The decoded
  weights are then of the size of the N(0, 0.02) bf16 weights above.
"""
from concurrent.futures import ThreadPoolExecutor
import math
import os

import numpy as np

H, I, E, TOP_K, LAYERS = 2816, 704, 128, 8, 30
GROUP = 16
SEED = 0

# key tags
_W, _ROUTER_W, _ROUTER_SCALE, _PES, _ZIPF, _X, _OUTLIER, _NORM, _INT4, _H1 = range(10)
GATE, UP, DOWN = 0, 1, 2

WORKLOADS = {
    0: dict(name="moe_layer_decode_T4", T=(4,), layers=1, zipf=False, outliers=False),
    1: dict(name="moe_layer_decode_T64", T=(64,), layers=1, zipf=False, outliers=False),
    2: dict(name="moe_layer_prefill_T2048_zipf1.2", T=(2048,), layers=1, zipf=True, outliers=False),
    3: dict(name="moe_30layer_decode_sweep_T1_T8", T=(1, 8), layers=30, zipf=False, outliers=False),
    4: dict(name="moe_layer_prefill_T16384_zipf1.2_outliers", T=(16384,), layers=1, zipf=True,
            outliers=True),
}


def _rng(seed, key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def f32_to_bf16_bits(a):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def proj_shape(proj, h=H, i=I):
    return (i, h) if proj in (GATE, UP) else (h, i)


def expert_weight(layer, proj, expert, seed=SEED, h=H, i=I):
    """One expert's projection weights as bf16 bits, shape [N, K]."""
    n, k = proj_shape(proj, h, i)
    rng = _rng(seed, (_W, layer, proj, expert))
    a = rng.standard_normal(n * k, dtype=np.float32)
    a *= np.float32(0.02)
    return f32_to_bf16_bits(a).reshape(n, k)


def _pool_size():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def expert_weights(layer, proj, experts=None, seed=SEED, h=H, i=I, e=E, out=None):
    """Stack of expert weights [len(experts), N, K] bf16 bits (threaded)."""
    experts = list(range(e)) if experts is None else list(experts)
    n, k = proj_shape(proj, h, i)
    if out is None:
        out = np.empty((len(experts), n, k), dtype=np.uint16)

    def one(j):
        out[j] = expert_weight(layer, proj, experts[j], seed, h, i)

    with ThreadPoolExecutor(_pool_size()) as ex:
        list(ex.map(one, range(len(experts))))
    return out


def router_params(layer, seed=SEED, h=H, e=E, zipf=False):
    """Router tensors for one layer: dict of bf16-bit arrays plus an optional
    float32 logit bias (None unless ``zipf``)."""
    w = _rng(seed, (_ROUTER_W, layer)).standard_normal(e * h) * h ** -0.5
    scale = _rng(seed, (_ROUTER_SCALE, layer)).uniform(0.8, 1.2, h)
    pes = _rng(seed, (_PES, layer)).uniform(0.5, 1.5, e)
    p = dict(w_router=f32_to_bf16_bits(w.astype(np.float32)).reshape(e, h),
             scale=f32_to_bf16_bits(scale.astype(np.float32)),
             per_expert_scale=f32_to_bf16_bits(pes.astype(np.float32)),
             bias=None)
    if zipf:
        sc = bf16_bits_to_f32(p["scale"]).astype(np.float64)
        sigma_l = h ** -0.5 * math.sqrt(float(np.mean(sc * sc)))
        beta = sigma_l * math.sqrt(6.0) / math.pi
        rank = _rng(seed, (_ZIPF, layer)).permutation(e) + 1
        p["bias"] = (-1.2 * beta * np.log(rank)).astype(np.float32)
    return p


def norm_weights(layer, seed=SEED, h=H):
    """The three learned norm weights of one layer's step after the sparse
    branch, bf16 bits [h] each ~ U(0.5, 1.5): pre_feedforward_layernorm_2 (the
    expert input), post_feedforward_layernorm_2 (the weighted expert sum) and
    post_feedforward_layernorm (the sum of the dense and sparse branches)."""
    return tuple(f32_to_bf16_bits(_rng(seed, (_NORM, layer, j)).uniform(0.5, 1.5, h).astype(np.float32))
                 for j in range(3))


def dense_branch_output(workload, t, seed=SEED, h=H):
    """A stand-in for the dense branch's normed output h1 [T, H] (the dense MLP
    is outside the block): bf16 bits ~ N(0, 1)."""
    a = _rng(seed, (_H1, workload, t)).standard_normal(t * h, dtype=np.float32).reshape(t, h)
    return f32_to_bf16_bits(a)


def activations(workload, t, seed=SEED, h=H, outliers=False):
    """x [T, H] bf16 bits ~ N(0, 1); with ``outliers`` ceil(0.01 T) rows x 20."""
    a = _rng(seed, (_X, workload, t)).standard_normal(t * h, dtype=np.float32).reshape(t, h)
    bits = f32_to_bf16_bits(a)
    if outliers and t > 0:
        n_out = math.ceil(0.01 * t)
        rows = _rng(seed, (_OUTLIER, workload, t)).choice(t, size=n_out, replace=False)
        v = bf16_bits_to_f32(bits[rows]) * np.float32(20.0)
        bits[rows] = f32_to_bf16_bits(v)
    return bits


def outlier_rows(workload, t, seed=SEED):
    n_out = math.ceil(0.01 * t)
    return np.sort(_rng(seed, (_OUTLIER, workload, t)).choice(t, size=n_out, replace=False))


def small_case(seed, t, h, i, e, k, zipf=False):
    """A self-contained small block (odd shapes for edge cases): returns bf16
    bits of x, router tensors and per-projection weight stacks [E, N, K]."""
    rng = _rng(seed, (99, t, h, i, e, k))
    x = f32_to_bf16_bits(rng.standard_normal((t, h)).astype(np.float32))
    w = f32_to_bf16_bits((rng.standard_normal((e, h)) * h ** -0.5).astype(np.float32))
    scale = f32_to_bf16_bits(rng.uniform(0.8, 1.2, h).astype(np.float32))
    pes = f32_to_bf16_bits(rng.uniform(0.5, 1.5, e).astype(np.float32))
    gate = f32_to_bf16_bits((rng.standard_normal((e, i, h)) * 0.02).astype(np.float32))
    up = f32_to_bf16_bits((rng.standard_normal((e, i, h)) * 0.02).astype(np.float32))
    down = f32_to_bf16_bits((rng.standard_normal((e, h, i)) * 0.02).astype(np.float32))
    bias = None
    if zipf:
        bias = (-1.2 * 0.02 * np.log(rng.permutation(e) + 1)).astype(np.float32)
    return dict(x=x, router=dict(w_router=w, scale=scale, per_expert_scale=pes, bias=bias),
                gate=gate, up=up, down=down)


# fp16 scale bytes per block of 32 weights of a row
INT4_SCALE_BYTES = {"q4_0": 2, "aff4": 4}


def _int4_draw(rng, fmt, n, k):
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    nb = k // 32
    if fmt == "q4_0":
        sc = rng.uniform(0.004, 0.008, (n, nb)).astype(np.float16)
    elif fmt == "aff4":
        sc = np.empty((n, nb, 2), dtype=np.float16)
        sc[..., 0] = rng.uniform(0.004, 0.008, (n, nb))
        sc[..., 1] = rng.uniform(-0.06, -0.035, (n, nb))
    else:
        raise ValueError(f"unknown int4 format {fmt}")
    return packed, np.ascontiguousarray(sc).view(np.uint8).reshape(n, -1)


def int4_expert(fmt, layer, proj, expert, seed=SEED, h=H, i=I):
    """One expert's int4 projection: (packed u8 [N, K/2], scale bytes u8
    [N, K/32 * INT4_SCALE_BYTES[fmt]]) -- fp16 d, or fp16 (s, b) pairs."""
    n, k = proj_shape(proj, h, i)
    return _int4_draw(_rng(seed, (_INT4, fmt == "aff4", layer, proj, expert)), fmt, n, k)


def int4_stack(fmt, layer, proj, seed=SEED, h=H, i=I, e=E):
    """int4_expert for experts 0..e-1, stacked: ([E, N, K/2], [E, N, ...])."""
    parts = [int4_expert(fmt, layer, proj, x, seed, h, i) for x in range(e)]
    return np.stack([p for p, _ in parts]), np.stack([s for _, s in parts])


def small_int4_case(seed, fmt, t, h, i, e, k, zipf=False):
    """small_case's x and router with int4 expert stacks (gate, up, down as
    (packed, scale bytes) pairs of [E, N, ...] arrays)."""
    c = small_case(seed, t, h, i, e, k, zipf)
    rng = _rng(seed, (_INT4, 99, fmt == "aff4", t, h, i, e, k))
    for name, (n, kk) in (("gate", (i, h)), ("up", (i, h)), ("down", (h, i))):
        parts = [_int4_draw(rng, fmt, n, kk) for _ in range(e)]
        c[name] = (np.stack([p for p, _ in parts]), np.stack([s for _, s in parts]))
    return c
