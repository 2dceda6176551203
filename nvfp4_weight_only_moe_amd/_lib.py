"""ctypes binding of libmoe_nvfp4.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks their
dtype, shape and contiguity, and passes raw pointers and the current HIP stream
to the C entry point of the same name.  All computation happens in the HIP
kernels; there is no fallback of any kind -- if the library is missing or a
call fails, an exception is raised.
"""
import ctypes
import os

import torch

from ._build import LIB as LIB_PATH

MOE_OK = 0
_ERRORS = {-1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_WORKSPACE",
           -4: "MOE_ERR_UNSUPPORTED", -5: "MOE_ERR_LAUNCH"}

EXPORTED = ("moe_route", "moe_route_bucket", "moe_route_bucket_prep", "moe_bucket",
            "moe_bucket_workspace_bytes", "nvfp4_expert_mlp", "nvfp4_expert_mlp_noalloc",
            "moe_layer_decode", "moe_layer_decode_workspace_bytes", "moe_layer_decode_error_offset",
            "nvfp4_expert_prep", "nvfp4_expert_gate_up", "nvfp4_expert_down",
            "moe_workspace_bytes", "moe_combine", "nvfp4_expert_prep_rmsnorm",
            "moe_combine_rmsnorm", "nvfp4_quantize", "nvfp4_repack",
            "nvfp4_dequant_bf16", "moe_dequant_f16", "moe_status_str", "moe_abi_version")

LAYOUT_CANONICAL, LAYOUT_TILED = 0, 1
# limits of moe_layer_decode (the three-launch decode path)
DECODE_MAX_TOKENS, DECODE_MAX_PAIRS, DECODE_MAX_HIDDEN = 8, 64, 4096
FORMAT_NVFP4, FORMAT_Q4_0, FORMAT_AFF4 = 0, 1, 2
FORMATS = {"nvfp4": FORMAT_NVFP4, "q4_0": FORMAT_Q4_0, "aff4": FORMAT_AFF4}
# scale bytes per 32 weights of a row: NVFP4 two E4M3 codes, Q4_0 one fp16 d,
# AFF4 one fp16 s and one fp16 b
SCALE_BYTES_PER_32 = {FORMAT_NVFP4: 2, FORMAT_Q4_0: 2, FORMAT_AFF4: 4}


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {status} ({_ERRORS.get(status, '?')}: "
                         f"{lib().moe_status_str(status).decode()})")


class Nvfp4TensorC(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_", ctypes.c_void_p), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("layout", ctypes.c_int32), ("format", ctypes.c_int32)]


_lib = None


def lib(path=None):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("MOE_NVFP4_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it first (python __graft_entry__.py build "
                           "or nvfp4_weight_only_moe_amd._build.build())")
    L = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    P = ctypes.POINTER(Nvfp4TensorC)
    sig = {
        "moe_route": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp]),
        "moe_bucket": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "moe_bucket_workspace_bytes": (sz, [i32, i32, i32]),
        "moe_route_bucket": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp,
                                            vp, vp, vp, vp, vp, sz, vp]),
        "moe_route_bucket_prep": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp,
                                                 vp, vp, vp, vp, vp, vp, sz, vp, f32, i32, vp, sz,
                                                 vp]),
        "nvfp4_expert_mlp": (ctypes.c_int, [vp, P, P, P, vp, vp, i32, i32, i32, i32, vp, vp, sz, vp]),
        "nvfp4_expert_mlp_noalloc": (ctypes.c_int, [vp, P, P, P, vp, vp, i32, i32, i32, i32, vp,
                                                    vp]),
        "nvfp4_expert_prep": (ctypes.c_int, [vp, i32, i32, i32, i32, i32, vp, sz, vp]),
        "moe_layer_decode": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, P, P, P,
                                            i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_layer_decode_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "moe_layer_decode_error_offset": (sz, [i32, i32, i32]),
        "nvfp4_expert_gate_up": (ctypes.c_int, [P, P, vp, vp, i32, i32, i32, i32, vp, sz, vp]),
        "nvfp4_expert_down": (ctypes.c_int, [P, vp, i32, i32, i32, i32, vp, vp, sz, vp]),
        "moe_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "moe_combine": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp, vp]),
        "nvfp4_expert_prep_rmsnorm": (ctypes.c_int, [vp, vp, f32, i32, i32, i32, i32, i32, vp, sz,
                                                     vp]),
        "moe_combine_rmsnorm": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, f32, f32, i32, i32, i32,
                                               vp, vp]),
        "nvfp4_quantize": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp]),
        "nvfp4_repack": (ctypes.c_int, [P, vp, vp, vp]),
        "nvfp4_dequant_bf16": (ctypes.c_int, [P, i32, vp, vp]),
        "moe_dequant_f16": (ctypes.c_int, [P, i32, vp, vp]),
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_abi_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status)


_B16 = (torch.bfloat16, torch.int16, torch.uint16)


class Nvfp4Weights:
    """One stack of 4-bit expert weights: packed [E,N,K/2] u8 codes, scales
    [E,N,K*SB/32] bytes (SB = SCALE_BYTES_PER_32[fmt]: NVFP4 E4M3 codes per 16,
    Q4_0 fp16 d per 32, AFF4 fp16 (s, b) per 32), global [E] f32 (NVFP4; None
    for the int4 formats), in the canonical or the tiled byte layout (same
    sizes)."""

    def __init__(self, packed, scales, global_scale, layout=LAYOUT_CANONICAL, fmt=FORMAT_NVFP4):
        if fmt not in SCALE_BYTES_PER_32:
            raise ValueError(f"unknown weight format {fmt}")
        self.packed, self.scales, self.global_scale = packed, scales, global_scale
        self.E, self.N, k2 = packed.shape
        self.K = 2 * k2
        self.layout = layout
        self.format = fmt

    @property
    def scale_bytes_per_row(self):
        return self.K * SCALE_BYTES_PER_32[self.format] // 32

    @classmethod
    def empty(cls, E, N, K, device="cuda", layout=LAYOUT_CANONICAL, fmt=FORMAT_NVFP4):
        sb = K * SCALE_BYTES_PER_32[fmt] // 32
        g = torch.empty((E,), dtype=torch.float32, device=device) if fmt == FORMAT_NVFP4 else None
        return cls(torch.empty((E, N, K // 2), dtype=torch.uint8, device=device),
                   torch.empty((E, N, sb), dtype=torch.uint8, device=device), g, layout, fmt)

    def c(self):
        _ptr(self.packed, torch.uint8, (self.E, self.N, self.K // 2), "packed")
        _ptr(self.scales, torch.uint8, (self.E, self.N, self.scale_bytes_per_row), "scales")
        if self.format == FORMAT_NVFP4 or self.global_scale is not None:
            _ptr(self.global_scale, torch.float32, (self.E,), "global")
        g = self.global_scale.data_ptr() if self.global_scale is not None else None
        return Nvfp4TensorC(self.packed.data_ptr(), self.scales.data_ptr(), g, self.E, self.N,
                            self.K, self.layout, self.format)

    def _g(self, f):
        return None if self.global_scale is None else f(self.global_scale)

    def select(self, e0, e1):
        """Experts e0..e1-1 (views, no copy)."""
        return Nvfp4Weights(self.packed[e0:e1], self.scales[e0:e1],
                            self._g(lambda g: g[e0:e1]), self.layout, self.format)

    def clone(self):
        return Nvfp4Weights(self.packed.clone(), self.scales.clone(), self._g(torch.clone),
                            self.layout, self.format)


def moe_route(x, w_router, router_scale, per_expert_scale, logit_bias, top_k, eps,
              topk_idx, topk_w, topk_w_raw, logits, stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    st = lib().moe_route(_ptr(x, _B16, (T, H), "x"), _ptr(w_router, _B16, (E, H), "w_router"),
                         _ptr(router_scale, _B16, (H,), "router_scale"),
                         _ptr(per_expert_scale, _B16, (E,), "per_expert_scale"),
                         _ptr(logit_bias, torch.float32, (E,), "logit_bias"), T, H, E, top_k,
                         float(eps), _ptr(topk_idx, torch.int32, (T, top_k), "topk_idx"),
                         _ptr(topk_w, torch.float32, (T, top_k), "topk_w"),
                         _ptr(topk_w_raw, torch.float32, (T, top_k), "topk_w_raw"),
                         _ptr(logits, torch.float32, (T, E), "logits"), _stream(stream))
    _check("moe_route", st)


def moe_route_bucket(x, w_router, router_scale, per_expert_scale, logit_bias, top_k, eps,
                     topk_idx, topk_w, topk_w_raw, logits, expert_offsets, sorted_pairs, pair_rank,
                     workspace, stream=None):
    """moe_route then moe_bucket in one call (same outputs)."""
    T, H = x.shape
    E = w_router.shape[0]
    st = lib().moe_route_bucket(
        _ptr(x, _B16, (T, H), "x"), _ptr(w_router, _B16, (E, H), "w_router"),
        _ptr(router_scale, _B16, (H,), "router_scale"),
        _ptr(per_expert_scale, _B16, (E,), "per_expert_scale"),
        _ptr(logit_bias, torch.float32, (E,), "logit_bias"), T, H, E, top_k, float(eps),
        _ptr(topk_idx, torch.int32, (T, top_k), "topk_idx"),
        _ptr(topk_w, torch.float32, (T, top_k), "topk_w"),
        _ptr(topk_w_raw, torch.float32, (T, top_k), "topk_w_raw"),
        _ptr(logits, torch.float32, (T, E), "logits"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(sorted_pairs, torch.int32, (T * top_k,), "sorted_pairs"),
        _ptr(pair_rank, torch.int32, (T * top_k,), "pair_rank"),
        _ptr(workspace, None, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("moe_route_bucket", st)


def moe_route_bucket_prep(x, w_router, router_scale, per_expert_scale, logit_bias, top_k, eps,
                          topk_idx, topk_w, topk_w_raw, logits, expert_offsets, sorted_pairs,
                          pair_rank, bucket_ws, norm_weight, norm_eps, I, expert_ws, stream=None):
    """moe_route_bucket, then nvfp4_expert_prep(x) (norm_weight None) or
    nvfp4_expert_prep_rmsnorm(x, norm_weight, norm_eps) into expert_ws."""
    T, H = x.shape
    E = w_router.shape[0]
    st = lib().moe_route_bucket_prep(
        _ptr(x, _B16, (T, H), "x"), _ptr(w_router, _B16, (E, H), "w_router"),
        _ptr(router_scale, _B16, (H,), "router_scale"),
        _ptr(per_expert_scale, _B16, (E,), "per_expert_scale"),
        _ptr(logit_bias, torch.float32, (E,), "logit_bias"), T, H, E, top_k, float(eps),
        _ptr(topk_idx, torch.int32, (T, top_k), "topk_idx"),
        _ptr(topk_w, torch.float32, (T, top_k), "topk_w"),
        _ptr(topk_w_raw, torch.float32, (T, top_k), "topk_w_raw"),
        _ptr(logits, torch.float32, (T, E), "logits"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(sorted_pairs, torch.int32, (T * top_k,), "sorted_pairs"),
        _ptr(pair_rank, torch.int32, (T * top_k,), "pair_rank"),
        _ptr(bucket_ws, None, None, "bucket_ws"), bucket_ws.numel() * bucket_ws.element_size(),
        _ptr(norm_weight, _B16, (H,), "norm_weight"), float(norm_eps), I,
        _ptr(expert_ws, None, None, "expert_ws"), expert_ws.numel() * expert_ws.element_size(),
        _stream(stream))
    _check("moe_route_bucket_prep", st)


def moe_bucket_workspace_bytes(T, top_k, E):
    return int(lib().moe_bucket_workspace_bytes(T, top_k, E))


def moe_bucket(topk_idx, E, expert_offsets, sorted_pairs, pair_rank, workspace, stream=None):
    T, top_k = topk_idx.shape
    st = lib().moe_bucket(_ptr(topk_idx, torch.int32, (T, top_k), "topk_idx"), T, top_k, E,
                          _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
                          _ptr(sorted_pairs, torch.int32, (T * top_k,), "sorted_pairs"),
                          _ptr(pair_rank, torch.int32, (T * top_k,), "pair_rank"),
                          _ptr(workspace, None, None, "workspace"), workspace.numel() * workspace.element_size(),
                          _stream(stream))
    _check("moe_bucket", st)


def moe_layer_decode_workspace_bytes(T, top_k, E, H, I):
    return int(lib().moe_layer_decode_workspace_bytes(T, top_k, E, H, I))


def moe_layer_decode_error_offset(T, top_k, E):
    return int(lib().moe_layer_decode_error_offset(T, top_k, E))


def decode_fits(T, top_k, H):
    """Whether moe_layer_decode takes this shape."""
    return 0 < T <= DECODE_MAX_TOKENS and T * top_k <= DECODE_MAX_PAIRS and H <= DECODE_MAX_HIDDEN


def moe_layer_decode(x, w_router, router_scale, per_expert_scale, logit_bias, top_k, eps, gate,
                     up, down, topk_idx, topk_w, topk_w_raw, expert_offsets, sorted_pairs,
                     pair_rank, out, workspace, stream=None):
    """The whole block for a decode batch (T <= 8) in three launches (up to
    32 pairs) or four."""
    T, H = x.shape
    E = w_router.shape[0]
    I = gate.N
    cg, cu, cd = gate.c(), up.c(), down.c()
    st = lib().moe_layer_decode(
        _ptr(x, _B16, (T, H), "x"), _ptr(w_router, _B16, (E, H), "w_router"),
        _ptr(router_scale, _B16, (H,), "router_scale"),
        _ptr(per_expert_scale, _B16, (E,), "per_expert_scale"),
        _ptr(logit_bias, torch.float32, (E,), "logit_bias"), T, H, E, top_k, float(eps),
        ctypes.byref(cg), ctypes.byref(cu), ctypes.byref(cd), I,
        _ptr(topk_idx, torch.int32, (T, top_k), "topk_idx"),
        _ptr(topk_w, torch.float32, (T, top_k), "topk_w"),
        _ptr(topk_w_raw, torch.float32, (T, top_k), "topk_w_raw"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(sorted_pairs, torch.int32, (T * top_k,), "sorted_pairs"),
        _ptr(pair_rank, torch.int32, (T * top_k,), "pair_rank"),
        _ptr(out, _B16, (T, H), "out"), _ptr(workspace, None, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("moe_layer_decode", st)


def moe_workspace_bytes(T, top_k, E, H, I):
    return int(lib().moe_workspace_bytes(T, top_k, E, H, I))


def nvfp4_expert_mlp(x_expert, gate, up, down, expert_offsets, sorted_pairs, top_k, y_sorted,
                     workspace, stream=None):
    T, H = x_expert.shape
    I = gate.N
    cg, cu, cd = gate.c(), up.c(), down.c()
    st = lib().nvfp4_expert_mlp(_ptr(x_expert, _B16, (T, H), "x_expert"), ctypes.byref(cg),
                                ctypes.byref(cu), ctypes.byref(cd),
                                _ptr(expert_offsets, torch.int32, (gate.E + 1,), "expert_offsets"),
                                _ptr(sorted_pairs, torch.int32, (T * top_k,), "sorted_pairs"), T,
                                top_k, H, I, _ptr(y_sorted, _B16, (T * top_k, H), "y_sorted"),
                                _ptr(workspace, None, None, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check("nvfp4_expert_mlp", st)


def nvfp4_expert_mlp_noalloc(x_expert, gate, up, down, expert_offsets, sorted_pairs, top_k,
                             y_sorted, stream=None):
    """nvfp4_expert_mlp on the library's own per-GPU scratch array (no
    workspace argument, nothing allocated); calls that overlap on one GPU race."""
    T, H = x_expert.shape
    I = gate.N
    cg, cu, cd = gate.c(), up.c(), down.c()
    st = lib().nvfp4_expert_mlp_noalloc(
        _ptr(x_expert, _B16, (T, H), "x_expert"), ctypes.byref(cg), ctypes.byref(cu),
        ctypes.byref(cd), _ptr(expert_offsets, torch.int32, (gate.E + 1,), "expert_offsets"),
        _ptr(sorted_pairs, torch.int32, (T * top_k,), "sorted_pairs"), T, top_k, H, I,
        _ptr(y_sorted, _B16, (T * top_k, H), "y_sorted"), _stream(stream))
    _check("nvfp4_expert_mlp_noalloc", st)


def nvfp4_expert_prep(x_expert, E, I, top_k, workspace, stream=None):
    """Stage 1 of the expert MLP; independent of the routing (may run beside
    moe_route / moe_bucket), must complete before nvfp4_expert_gate_up."""
    T, H = x_expert.shape
    st = lib().nvfp4_expert_prep(_ptr(x_expert, _B16, (T, H), "x_expert"), T, top_k, E, H, I,
                                 _ptr(workspace, None, None, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check("nvfp4_expert_prep", st)


def nvfp4_expert_prep_rmsnorm(x, norm_weight, eps, E, I, top_k, workspace, stream=None):
    """nvfp4_expert_prep with the learned RMSNorm of x as the expert input."""
    T, H = x.shape
    st = lib().nvfp4_expert_prep_rmsnorm(_ptr(x, _B16, (T, H), "x"),
                                         _ptr(norm_weight, _B16, (H,), "norm_weight"), float(eps),
                                         T, top_k, E, H, I, _ptr(workspace, None, None, "workspace"),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(stream))
    _check("nvfp4_expert_prep_rmsnorm", st)


def nvfp4_expert_gate_up(gate, up, expert_offsets, sorted_pairs, T, top_k, H, workspace,
                         stream=None):
    cg, cu = gate.c(), up.c()
    st = lib().nvfp4_expert_gate_up(ctypes.byref(cg), ctypes.byref(cu),
                                    _ptr(expert_offsets, torch.int32, (gate.E + 1,), "expert_offsets"),
                                    _ptr(sorted_pairs, torch.int32, (T * top_k,), "sorted_pairs"),
                                    T, top_k, H, gate.N, _ptr(workspace, None, None, "workspace"),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check("nvfp4_expert_gate_up", st)


def nvfp4_expert_down(down, expert_offsets, T, top_k, y_sorted, workspace, stream=None):
    cd = down.c()
    st = lib().nvfp4_expert_down(ctypes.byref(cd),
                                 _ptr(expert_offsets, torch.int32, (down.E + 1,), "expert_offsets"),
                                 T, top_k, down.N, down.K,
                                 _ptr(y_sorted, _B16, (T * top_k, down.N), "y_sorted"),
                                 _ptr(workspace, None, None, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check("nvfp4_expert_down", st)


def moe_combine(y_sorted, topk_w, pair_rank, out, stream=None):
    T, top_k = topk_w.shape
    H = out.shape[1]
    st = lib().moe_combine(_ptr(y_sorted, _B16, (T * top_k, H), "y_sorted"),
                           _ptr(topk_w, torch.float32, (T, top_k), "topk_w"),
                           _ptr(pair_rank, torch.int32, (T * top_k,), "pair_rank"), T, top_k, H,
                           _ptr(out, _B16, (T, H), "out"), _stream(stream))
    _check("moe_combine", st)


def moe_combine_rmsnorm(y_sorted, topk_w, pair_rank, post_norm2, eps, out, h1=None,
                        post_norm=None, residual=None, layer_scalar=1.0, stream=None):
    """h2 = rmsnorm(sum_j w_j y_j, post_norm2); with post_norm:
    out = (residual + rmsnorm(h1 + h2, post_norm)) * layer_scalar (h1 None:
    zero), else out = h2."""
    T, top_k = topk_w.shape
    H = out.shape[1]
    opt = lambda t, n: None if t is None else _ptr(t, _B16, (T, H), n)
    st = lib().moe_combine_rmsnorm(_ptr(y_sorted, _B16, (T * top_k, H), "y_sorted"),
                                   _ptr(topk_w, torch.float32, (T, top_k), "topk_w"),
                                   _ptr(pair_rank, torch.int32, (T * top_k,), "pair_rank"),
                                   _ptr(post_norm2, _B16, (H,), "post_norm2"), opt(h1, "h1"),
                                   _ptr(post_norm, _B16, (H,), "post_norm"),
                                   opt(residual, "residual"), float(eps), float(layer_scalar), T,
                                   top_k, H, _ptr(out, _B16, (T, H), "out"), _stream(stream))
    _check("moe_combine_rmsnorm", st)


def nvfp4_quantize(w, out, stream=None):
    """w [E, N, K] bf16 -> out (Nvfp4Weights of the same shape)."""
    E, N, K = w.shape
    st = lib().nvfp4_quantize(_ptr(w, _B16, (E, N, K), "w"), E, N, K,
                              _ptr(out.packed, torch.uint8, (E, N, K // 2), "packed"),
                              _ptr(out.scales, torch.uint8, (E, N, K // 16), "scales"),
                              _ptr(out.global_scale, torch.float32, (E,), "global"), _stream(stream))
    _check("nvfp4_quantize", st)


def nvfp4_repack(w, stream=None):
    """Canonical -> tiled copy of a stack (the layout the expert kernels read)."""
    if w.layout != LAYOUT_CANONICAL:
        raise ValueError("nvfp4_repack takes canonical weights")
    out = Nvfp4Weights(torch.empty_like(w.packed), torch.empty_like(w.scales), w.global_scale,
                       LAYOUT_TILED, w.format)
    c = w.c()
    st = lib().nvfp4_repack(ctypes.byref(c), _ptr(out.packed, torch.uint8, None, "packed"),
                            _ptr(out.scales, torch.uint8, None, "scales"), _stream(stream))
    _check("nvfp4_repack", st)
    return out


def nvfp4_dequant_bf16(w, e, out, stream=None):
    c = w.c()
    st = lib().nvfp4_dequant_bf16(ctypes.byref(c), e, _ptr(out, _B16, (w.N, w.K), "out"),
                                  _stream(stream))
    _check("nvfp4_dequant_bf16", st)


def moe_dequant_f16(w, e, out, stream=None):
    """The f16 weights the expert kernels multiply for expert e (any format
    and layout; NVFP4 without its FP32 tensor scale)."""
    c = w.c()
    st = lib().moe_dequant_f16(ctypes.byref(c), e,
                               _ptr(out, (torch.float16, torch.int16, torch.uint16), (w.N, w.K),
                                    "out"), _stream(stream))
    _check("moe_dequant_f16", st)
