"""The MoE expert block in float64 (oracle; test infrastructure only).

"Gemma 4 26B-A4B (MoE) - Core AI", Architecture: every layer runs a sparse
branch beside its dense MLP; the router reads the raw residual and the experts
read the residual after their own pre-norm; the routed outputs are summed with
the routing weights.  Router: RMSNorm without a learned scale -> times a
learned per-channel ``scale`` and hidden^-0.5 -> linear to the 128 experts ->
softmax in fp32 over all experts -> top-8 -> renormalise to sum 1 -> times a
learned ``per_expert_scale`` gathered at the chosen ids.  Experts are
GELU-gated with the tanh form of GELU: A = gelu_tanh(x Wg^T) * (x Wu^T),
y = A Wd^T (gate and up 2816 -> 704, down 704 -> 2816; same page,
Architecture table and New source modules).  Sort-by-expert bucketing is the
grouped-GEMM form the same page names under "Decode only".

Readings (the pages leave these open):
* RMSNorm epsilon 1e-6, added to mean(x^2) inside the square root.
* ``scale`` is a per-channel vector; no rounding anywhere before the logits
  (this oracle works in float64 throughout).
* An optional per-expert logit bias (zero on the pages) is added to the logits;
  it is how synthetic inputs get a skewed expert popularity.
* Top-k ties go to the lower expert id; the order of the k ids is not part of
  the result (compared as sets).
* The bucket order is (expert, token, slot); the routing weight multiplies the
  expert output after the down projection.
* The learned norms of the layer step (``pre_feedforward_layernorm_2`` on the
  expert input, ``post_feedforward_layernorm_2`` on the weighted sum,
  ``post_feedforward_layernorm`` on the sum of the dense branch's h1 and the
  sparse branch's h2) are RMSNorms with a multiplicative per-channel weight and
  the same epsilon; a checkpoint that stores the weight as an offset from 1
  passes 1 + w.  The layer's dense MLP is not part of the block: its output h1
  (after ``post_feedforward_layernorm_1``) is an input of ``sparse_branch``
  (zero when absent).
"""
import numpy as np

from .formats import dequantize

SQRT_2_OVER_PI = np.sqrt(2.0 / np.pi)


def gelu_tanh(x):
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))  (Hendrycks & Gimpel)."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(SQRT_2_OVER_PI * (x + 0.044715 * x ** 3)))


def router_logits(x, w_router, scale, bias=None, eps=1e-6):
    """logits[t, e] = (x_t / sqrt(mean(x_t^2) + eps) * scale * H^-0.5) . W[e] (+ b_e)."""
    x = np.asarray(x, np.float64)
    h = x.shape[-1]
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    r = x / rms * np.asarray(scale, np.float64) * h ** -0.5
    logits = r @ np.asarray(w_router, np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)
    return logits


def softmax(logits):
    z = logits - logits.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


def topk_ids(logits, k):
    """Top-k expert ids per token by logit, ties to the lower id; sorted by
    (logit descending, id ascending)."""
    t, e = logits.shape
    out = np.empty((t, k), dtype=np.int64)
    for i in range(t):
        order = sorted(range(e), key=lambda j: (-logits[i, j], j))
        out[i] = order[:k]
    return out


def route(x, w_router, scale, per_expert_scale, k=8, bias=None, eps=1e-6, tie_band=1e-6):
    """The router.  Returns a dict with
    idx [T,k] int64, w [T,k] (after per_expert_scale), w_raw [T,k] (sum 1),
    logits [T,E], probs [T,E], near_tie [T] bool (l_(k) - l_(k+1) < tie_band),
    band: list of sets {e : |l_e - l_(k)| < tie_band}."""
    logits = router_logits(x, w_router, scale, bias, eps)
    probs = softmax(logits)
    idx = topk_ids(logits, k)
    sel = np.take_along_axis(probs, idx, axis=1)
    w_raw = sel / sel.sum(axis=1, keepdims=True)
    pes = np.asarray(per_expert_scale, np.float64)
    w = w_raw * pes[idx]
    t, e = logits.shape
    near = np.zeros(t, dtype=bool)
    band = []
    for i in range(t):
        srt = np.sort(logits[i])[::-1]
        lk = srt[k - 1]
        nxt = srt[k] if k < e else -np.inf
        near[i] = (lk - nxt) < tie_band
        band.append(set(np.nonzero(np.abs(logits[i] - lk) < tie_band)[0].tolist()))
    return dict(idx=idx, w=w, w_raw=w_raw, logits=logits, probs=probs, near_tie=near, band=band)


def weights_for_ids(logits, per_expert_scale, ids):
    """Routing weights for a given id set per token: softmax probabilities at
    the ids, renormalised to sum 1, times per_expert_scale."""
    probs = softmax(np.asarray(logits, np.float64))
    sel = np.take_along_axis(probs, ids, axis=1)
    w_raw = sel / sel.sum(axis=1, keepdims=True)
    return w_raw * np.asarray(per_expert_scale, np.float64)[ids], w_raw


def bucket(idx, num_experts):
    """Sort the T*k (token, slot) pairs by (expert, token, slot).

    Returns counts [E], offsets [E+1], sorted_pairs [P] (pair id p = t*k + j),
    pair_rank [P] (position of pair p in the sorted order)."""
    idx = np.asarray(idx)
    t, k = idx.shape
    pairs = [(int(idx[i, j]), i, j) for i in range(t) for j in range(k)]
    order = sorted(pairs)
    sorted_pairs = np.array([i * k + j for (_, i, j) in order], dtype=np.int64)
    counts = np.zeros(num_experts, dtype=np.int64)
    for (e, _, _) in pairs:
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    pair_rank = np.empty(t * k, dtype=np.int64)
    pair_rank[sorted_pairs] = np.arange(t * k)
    return dict(counts=counts, offsets=offsets, sorted_pairs=sorted_pairs, pair_rank=pair_rank)


def expert_mlp(x_rows, wg, wu, wd):
    """One expert on its rows: (gelu_tanh(X Wg^T) * (X Wu^T)) Wd^T, all float64."""
    g = x_rows @ wg.T
    u = x_rows @ wu.T
    return (gelu_tanh(g) * u) @ wd.T


def experts(x_expert, buckets, top_k, gate, up, down, only_pairs=None):
    """Expert outputs for every sorted pair: Y [P, H] float64 in sorted order.

    gate/up/down are callables ``e -> float64 [N, K]`` returning the dequantised
    weights of expert e (so only touched experts are decoded).  ``only_pairs``
    (optional set of sorted positions) restricts the work to those rows; the
    other rows of Y are left NaN."""
    x_expert = np.asarray(x_expert, np.float64)
    offs = buckets["offsets"]
    sp = buckets["sorted_pairs"]
    y = np.full((len(sp), x_expert.shape[1]), np.nan)
    for e in range(len(offs) - 1):
        lo, hi = int(offs[e]), int(offs[e + 1])
        rows = [r for r in range(lo, hi) if only_pairs is None or r in only_pairs]
        if not rows:
            continue
        toks = sp[rows] // top_k
        y[rows] = expert_mlp(x_expert[toks], gate(e), up(e), down(e))
    return y


def combine(y_sorted, w, pair_rank, top_k):
    """out[t] = sum_j w[t, j] * Y[pair_rank[t*k + j]]   (float64)."""
    t = w.shape[0]
    out = np.zeros((t, y_sorted.shape[1]))
    for i in range(t):
        for j in range(top_k):
            out[i] += w[i, j] * y_sorted[pair_rank[i * top_k + j]]
    return out


def nvfp4_weights(packed, scales, gscale):
    """Callable e -> dequantised float64 [N, K] for one projection stack."""
    def get(e):
        return dequantize(packed[e], scales[e], gscale[e])
    return get


def moe_block(x, x_expert, router, gate, up, down, k=8, eps=1e-6, ids=None):
    """Router -> bucketing -> experts -> weighted sum (float64).

    router: dict(w_router [E,H], scale [H], per_expert_scale [E], bias [E]|None)
    gate/up/down: callables e -> dequantised weights.  ``ids`` optionally forces
    the expert set per token (used to follow a near-tie choice of the GPU)."""
    r = route(x, router["w_router"], router["scale"], router["per_expert_scale"], k,
              router.get("bias"), eps)
    if ids is not None:
        w, w_raw = weights_for_ids(r["logits"], router["per_expert_scale"], np.asarray(ids))
        r = dict(r, idx=np.asarray(ids), w=w, w_raw=w_raw)
    e = np.asarray(router["w_router"]).shape[0]
    b = bucket(r["idx"], e)
    y = experts(x_expert, b, k, gate, up, down)
    out = combine(y, r["w"], b["pair_rank"], k)
    return dict(out=out, route=r, buckets=b, y_sorted=y)


def moe_block_dense(x, x_expert, router, gate, up, down, k=8, eps=1e-6):
    """The same block written as the dense "over-read" the Core AI page
    describes for a missing gather kernel: every expert runs on every token,
    then a [T, E] routing mask (zero off the top-k) mixes the outputs.  It
    shares no bucketing or combine code with ``moe_block``."""
    r = route(x, router["w_router"], router["scale"], router["per_expert_scale"], k,
              router.get("bias"), eps)
    xe = np.asarray(x_expert, np.float64)
    t = xe.shape[0]
    e_num = np.asarray(router["w_router"]).shape[0]
    mask = np.zeros((t, e_num))
    for i in range(t):
        for j in range(k):
            mask[i, r["idx"][i, j]] += r["w"][i, j]
    out = None
    for e in range(e_num):
        ye = expert_mlp(xe, gate(e), up(e), down(e))
        contrib = mask[:, e:e + 1] * ye
        out = contrib if out is None else out + contrib
    return out


def rms_norm(x, weight, eps=1e-6):
    """Learned RMSNorm of each row (float64): x / sqrt(mean(x^2) + eps) * weight.

    "Gemma 4 26B-A4B (MoE) - Core AI", Architecture code sketch: the experts
    read pre_feedforward_layernorm_2(residual); the weighted expert sum goes
    through post_feedforward_layernorm_2."""
    x = np.asarray(x, np.float64)
    inv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * inv * np.asarray(weight, np.float64)


def sparse_branch(residual, router, pre_norm2, post_norm2, gate, up, down, k=8, eps=1e-6,
                  ids=None, post_norm=None, h1=None, layer_scalar=1.0):
    """The sparse branch and the layer step that follows it (float64), same
    page, Architecture code sketch:

        w, idx = router(residual)                      # the RAW residual
        h2 = experts(rms_norm(residual, pre_norm2), idx)
        h2 = rms_norm(sum_k w_k h2_k, post_norm2)
        x  = residual + rms_norm(h1 + h2, post_norm)   # h1: the dense branch
        x  = x * layer_scalar

    ``h1`` is the dense branch's output (None: zero).  Without ``post_norm``
    the layer step is not taken and ``out`` is None.  Returns dict(out, h2,
    x_expert, block)."""
    res = np.asarray(residual, np.float64)
    x_expert = rms_norm(res, pre_norm2, eps)
    blk = moe_block(res, x_expert, router, gate, up, down, k, eps, ids)
    h2 = rms_norm(blk["out"], post_norm2, eps)
    out = None
    if post_norm is not None:
        u = h2 if h1 is None else np.asarray(h1, np.float64) + h2
        out = (res + rms_norm(u, post_norm, eps)) * layer_scalar
    return dict(out=out, h2=h2, x_expert=x_expert, block=blk)
