"""CPU checks of the C ABI: the built library loads, exports every function
the header declares, and rejects bad arguments with the documented status
codes before queueing any GPU work (no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def L():
    from nvfp4_weight_only_moe_amd import _build, _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    return _lib.lib()


def test_header_declares_the_hot_path():
    names = _declared()
    for n in ("moe_route", "moe_bucket", "moe_route_bucket", "nvfp4_expert_mlp", "moe_combine"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    from nvfp4_weight_only_moe_amd._lib import EXPORTED
    names = _declared()
    assert set(names) == set(EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    for st in (0, -1, -2, -3, -4, -5):
        assert L.moe_status_str(st)
    assert L.moe_abi_version() >> 16 == 3


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation
NULL = None


def test_route_rejects(L):
    args = [FAKE, FAKE, FAKE, FAKE, NULL, 4, 2816, 128, 8, 1e-6, FAKE, FAKE, NULL, FAKE, NULL]
    a = list(args); a[0] = NULL
    assert L.moe_route(*a) == -1                      # x NULL with T > 0
    a = list(args); a[11] = NULL
    assert L.moe_route(*a) == -1                      # topk_w required (logits may be NULL)
    a = list(args); a[13], a[6] = NULL, 2800
    assert L.moe_route(*a) == -2                      # checked without logits too
    a = list(args); a[6] = 2800
    assert L.moe_route(*a) == -2                      # H % 64
    a = list(args); a[8] = 129
    assert L.moe_route(*a) == -2                      # top_k > E
    a = list(args); a[7] = 120
    assert L.moe_route(*a) == -4                      # E % 16
    a = list(args); a[7], a[8] = 512, 8
    assert L.moe_route(*a) == -4                      # E > 256
    a = list(args); a[5] = -1
    assert L.moe_route(*a) == -2


def test_bucket_rejects(L):
    ws = L.moe_bucket_workspace_bytes(64, 8, 128)
    assert ws >= 256
    assert L.moe_bucket(FAKE, 64, 8, 128, FAKE, FAKE, FAKE, FAKE, ws - 1, NULL) == -3
    assert L.moe_bucket(FAKE, 64, 8, 128, FAKE, FAKE, FAKE, NULL, ws, NULL) == -1
    assert L.moe_bucket(FAKE, 64, 17, 128, FAKE, FAKE, FAKE, FAKE, ws, NULL) == -4
    assert L.moe_bucket(FAKE, 64, 8, 300, FAKE, FAKE, FAKE, FAKE, ws, NULL) == -4
    assert L.moe_bucket(FAKE, -2, 8, 128, FAKE, FAKE, FAKE, FAKE, ws, NULL) == -2


def test_route_bucket_rejects(L):
    ws = L.moe_bucket_workspace_bytes(64, 8, 128)
    args = [FAKE, FAKE, FAKE, FAKE, NULL, 64, 2816, 128, 8, 1e-6, FAKE, FAKE, NULL, FAKE,
            FAKE, FAKE, FAKE, FAKE, ws, NULL]
    assert L.moe_route_bucket(*args[:18], ws - 1, NULL) == -3   # bucket workspace too small
    a = list(args); a[17] = NULL
    assert L.moe_route_bucket(*a) == -1                          # workspace NULL
    a = list(args); a[15] = NULL
    assert L.moe_route_bucket(*a) == -1                          # sorted_pairs NULL with T > 0
    a = list(args); a[6] = 2800
    assert L.moe_route_bucket(*a) == -2                          # H % 64
    a = list(args); a[7] = 120
    assert L.moe_route_bucket(*a) == -4                          # E % 16
    a = list(args); a[8] = 17
    assert L.moe_route_bucket(*a) == -4                          # top_k > 16
    a = list(args); a[5] = -1
    assert L.moe_route_bucket(*a) == -2


def _tensor(E, N, K, layout=1, fmt=0, glob=0x3000):
    from nvfp4_weight_only_moe_amd._lib import Nvfp4TensorC
    return Nvfp4TensorC(0x1000, 0x2000, glob, E, N, K, layout, fmt)


def test_expert_mlp_rejects(L):
    T, k, E, H, I = 64, 8, 128, 2816, 704
    ws = L.moe_workspace_bytes(T, k, E, H, I)
    g, u, d = _tensor(E, I, H), _tensor(E, I, H), _tensor(E, H, I)
    ok = [FAKE, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), FAKE, FAKE, T, k, H, I, FAKE, FAKE, ws, NULL]
    a = list(ok); a[12] = ws - 1
    assert L.nvfp4_expert_mlp(*a) == -3
    a = list(ok); a[11] = NULL
    assert L.nvfp4_expert_mlp(*a) == -1
    bad_d = _tensor(E, H, I + 64)
    a = list(ok); a[3] = ctypes.byref(bad_d)
    assert L.nvfp4_expert_mlp(*a) == -2
    a = list(ok); a[9] = I + 32
    g2, u2, d2 = _tensor(E, I + 32, H), _tensor(E, I + 32, H), _tensor(E, H, I + 32)
    a[1], a[2], a[3] = ctypes.byref(g2), ctypes.byref(u2), ctypes.byref(d2)
    a[12] = L.moe_workspace_bytes(T, k, E, H, I + 32)
    assert L.nvfp4_expert_mlp(*a) == -4               # I % 64
    nul = _tensor(E, I, H); nul.scales = None
    a = list(ok); a[1] = ctypes.byref(nul)
    assert L.nvfp4_expert_mlp(*a) == -1
    canon = _tensor(E, I, H, layout=0)                # the kernels read the tiled layout
    a = list(ok); a[2] = ctypes.byref(canon)
    assert L.nvfp4_expert_mlp(*a) == -4
    # stage calls validate the same way
    assert L.nvfp4_expert_prep(FAKE, T, k, E, H, I, FAKE, ws - 1, NULL) == -3
    assert L.nvfp4_expert_prep(NULL, T, k, E, H, I, FAKE, ws, NULL) == -1
    assert L.nvfp4_expert_prep(FAKE, T, k, E, H, I, NULL, ws, NULL) == -1
    assert L.nvfp4_expert_prep(FAKE, T, k, E, H + 32, I, FAKE, ws, NULL) == -4
    assert L.nvfp4_expert_gate_up(ctypes.byref(g), ctypes.byref(d), FAKE, FAKE, T, k, H, I, FAKE, ws, NULL) == -2
    assert L.nvfp4_expert_down(ctypes.byref(d), FAKE, T, k, H, I, NULL, FAKE, ws, NULL) == -1


def test_combine_quantize_dequant_reject(L):
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 8, 2812, FAKE, NULL) == -2
    assert L.moe_combine(NULL, FAKE, FAKE, 4, 8, 2816, FAKE, NULL) == -1
    assert L.nvfp4_quantize(FAKE, 1, 16, 48, FAKE, FAKE, FAKE, NULL) == -2
    assert L.nvfp4_quantize(FAKE, 1, 16, 64, FAKE, NULL, FAKE, NULL) == -1
    t = _tensor(2, 16, 64)
    assert L.nvfp4_dequant_bf16(ctypes.byref(t), 2, FAKE, NULL) == -2
    assert L.nvfp4_dequant_bf16(ctypes.byref(t), 0, NULL, NULL) == -1
    t7 = _tensor(2, 16, 64, layout=7)
    assert L.nvfp4_dequant_bf16(ctypes.byref(t7), 0, FAKE, NULL) == -4
    t24 = _tensor(2, 24, 64, layout=1)
    assert L.nvfp4_dequant_bf16(ctypes.byref(t24), 0, FAKE, NULL) == -2   # tiled needs N % 16
    c = _tensor(2, 16, 64, layout=0)
    assert L.nvfp4_repack(ctypes.byref(c), NULL, FAKE, NULL) == -1
    assert L.nvfp4_repack(ctypes.byref(_tensor(2, 16, 64, layout=1)), FAKE, FAKE, NULL) == -4
    assert L.nvfp4_repack(ctypes.byref(_tensor(2, 20, 64, layout=0)), FAKE, FAKE, NULL) == -2


def test_norm_entry_points_reject(L):
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 17, 2816, FAKE, NULL) == -4        # top_k > 16
    # moe_combine_rmsnorm(y, w, rank, norm2_w, h1, norm_w, residual, eps, scalar, T, k, H,
    #                     out, stream)
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, 1.0, 4, 8, 2816, FAKE, NULL]
    a = list(ok); a[3] = NULL
    assert L.moe_combine_rmsnorm(*a) == -1                                      # norm2 weight
    a = list(ok); a[6] = NULL
    assert L.moe_combine_rmsnorm(*a) == -1                                      # residual for the step
    a = list(ok); a[5] = NULL
    assert L.moe_combine_rmsnorm(*a) == -2                                      # h1/residual without the step
    a = list(ok); a[5], a[6] = NULL, NULL
    assert L.moe_combine_rmsnorm(*a) == -2                                      # h1 without the step
    a = list(ok); a[7] = -1.0
    assert L.moe_combine_rmsnorm(*a) == -2                                      # eps < 0
    a = list(ok); a[7] = float("nan")
    assert L.moe_combine_rmsnorm(*a) == -2
    a = list(ok); a[11] = 8200
    assert L.moe_combine_rmsnorm(*a) == -4                                      # H > 8192
    a = list(ok); a[11] = 2812
    assert L.moe_combine_rmsnorm(*a) == -2                                      # H % 8
    a = list(ok); a[10] = 17
    assert L.moe_combine_rmsnorm(*a) == -4                                      # top_k > 16
    a = list(ok); a[9] = 0
    assert L.moe_combine_rmsnorm(*a) == 0                                       # T = 0: no-op
    # nvfp4_expert_prep_rmsnorm(x, norm_w, eps, T, k, E, H, I, ws, ws_bytes, stream)
    ws = L.moe_workspace_bytes(4, 8, 128, 2816, 704)
    ok = [FAKE, FAKE, 1e-6, 4, 8, 128, 2816, 704, FAKE, ws, NULL]
    a = list(ok); a[1] = NULL
    assert L.nvfp4_expert_prep_rmsnorm(*a) == -1
    a = list(ok); a[0] = NULL
    assert L.nvfp4_expert_prep_rmsnorm(*a) == -1
    a = list(ok); a[2] = -0.5
    assert L.nvfp4_expert_prep_rmsnorm(*a) == -2
    a = list(ok); a[9] = ws - 1
    assert L.nvfp4_expert_prep_rmsnorm(*a) == -3


def test_workspace_sizes_cover_buffers(L):
    T, k, E, H, I = 16384, 8, 128, 2816, 704
    P = T * k
    ws = L.moe_workspace_bytes(T, k, E, H, I)
    assert ws >= T * H * 2 + P * I * 2 + P * 4 + T * 4
    assert L.moe_workspace_bytes(0, k, E, H, I) > 0
    assert L.moe_bucket_workspace_bytes(T, k, E) >= 256


def test_weight_format_checks(L):
    """Formats: unknown ones are rejected, gate and up must agree, the FP32
    global may be NULL for the int4 formats only (T = 0: nothing launched)."""
    T, k, E, H, I = 64, 8, 128, 2816, 704
    ws = L.moe_workspace_bytes(T, k, E, H, I)
    R = ctypes.byref
    for fmt in (1, 2):
        g, u, d = (_tensor(E, I, H, fmt=fmt, glob=None), _tensor(E, I, H, fmt=fmt, glob=None),
                   _tensor(E, H, I, fmt=fmt, glob=None))
        assert L.nvfp4_expert_gate_up(R(g), R(u), FAKE, FAKE, 0, k, H, I, FAKE, ws, NULL) == 0
        assert L.nvfp4_expert_down(R(d), FAKE, 0, k, H, I, FAKE, FAKE, ws, NULL) == 0
        assert L.nvfp4_expert_mlp(FAKE, R(g), R(u), R(d), FAKE, FAKE, 0, k, H, I, FAKE, FAKE, ws,
                                  NULL) == 0
    g0 = _tensor(E, I, H, fmt=0, glob=None)                      # NVFP4 needs its global
    assert L.nvfp4_expert_gate_up(R(g0), R(g0), FAKE, FAKE, 0, k, H, I, FAKE, ws, NULL) == -1
    q, a = _tensor(E, I, H, fmt=1), _tensor(E, I, H, fmt=2)
    assert L.nvfp4_expert_gate_up(R(q), R(a), FAKE, FAKE, T, k, H, I, FAKE, ws, NULL) == -4
    assert L.nvfp4_expert_mlp(FAKE, R(q), R(a), R(_tensor(E, H, I, fmt=1)), FAKE, FAKE, T, k, H,
                              I, FAKE, FAKE, ws, NULL) == -4
    bad = _tensor(E, I, H, fmt=3)
    assert L.nvfp4_expert_gate_up(R(bad), R(bad), FAKE, FAKE, T, k, H, I, FAKE, ws, NULL) == -4
    assert L.nvfp4_expert_down(R(_tensor(E, H, I, fmt=-1)), FAKE, T, k, H, I, FAKE, FAKE, ws,
                               NULL) == -4
    # mixed formats across gate/up and down are allowed (T = 0)
    assert L.nvfp4_expert_mlp(FAKE, R(q), R(q), R(_tensor(E, H, I, fmt=2)), FAKE, FAKE, 0, k, H,
                              I, FAKE, FAKE, ws, NULL) == 0
    # dequant / repack
    assert L.moe_dequant_f16(R(_tensor(2, 16, 64, fmt=3)), 0, FAKE, NULL) == -4
    assert L.moe_dequant_f16(R(_tensor(2, 16, 64, fmt=1, glob=None)), 2, FAKE, NULL) == -2
    assert L.moe_dequant_f16(R(_tensor(2, 16, 64, fmt=2, glob=None)), 0, NULL, NULL) == -1
    assert L.nvfp4_dequant_bf16(R(_tensor(2, 16, 64, fmt=1)), 0, FAKE, NULL) == -4
    assert L.nvfp4_repack(R(_tensor(2, 16, 64, layout=0, fmt=4)), FAKE, FAKE, NULL) == -4


def test_route_bucket_prep_rejects(L):
    T, k, E, H, I = 64, 8, 128, 2816, 704
    wsb = L.moe_bucket_workspace_bytes(T, k, E)
    wse = L.moe_workspace_bytes(T, k, E, H, I)
    # (x, w, scale, pes, bias, T, H, E, k, eps, idx, w, w_raw, logits, off, sp, pr,
    #  bucket_ws, bucket_ws_bytes, norm_w, norm_eps, I, expert_ws, expert_ws_bytes, stream)
    ok = [FAKE, FAKE, FAKE, FAKE, NULL, T, H, E, k, 1e-6, FAKE, FAKE, NULL, FAKE, FAKE, FAKE,
          FAKE, FAKE, wsb, NULL, 0.0, I, FAKE, wse, NULL]
    a = list(ok); a[18] = wsb - 1
    assert L.moe_route_bucket_prep(*a) == -3                 # bucket workspace
    a = list(ok); a[23] = wse - 1
    assert L.moe_route_bucket_prep(*a) == -3                 # expert workspace
    a = list(ok); a[22] = NULL
    assert L.moe_route_bucket_prep(*a) == -1
    a = list(ok); a[19], a[20] = FAKE, -1.0
    assert L.moe_route_bucket_prep(*a) == -2                 # norm eps < 0
    a = list(ok); a[21] = I + 32
    a[23] = L.moe_workspace_bytes(T, k, E, H, I + 32)
    assert L.moe_route_bucket_prep(*a) == -4                 # I % 64
    a = list(ok); a[0] = NULL
    assert L.moe_route_bucket_prep(*a) == -1                 # x NULL with T > 0
    a = list(ok); a[7] = 120
    assert L.moe_route_bucket_prep(*a) == -4                 # E % 16


def test_layer_decode_rejects(L):
    T, k, E, H, I = 8, 8, 128, 2816, 704
    ws = L.moe_layer_decode_workspace_bytes(T, k, E, H, I)
    assert ws >= L.moe_workspace_bytes(T, k, E, H, I) + T * E * 4
    assert L.moe_layer_decode_error_offset(T, k, E) >= T * E * 4
    R = ctypes.byref
    g, u, d = _tensor(E, I, H), _tensor(E, I, H), _tensor(E, H, I)
    # (x, w, scale, pes, bias, T, H, E, k, eps, gate, up, down, I, idx, w, w_raw, off, sp, pr,
    #  out, ws, ws_bytes, stream)
    ok = [FAKE, FAKE, FAKE, FAKE, NULL, T, H, E, k, 1e-6, R(g), R(u), R(d), I, FAKE, FAKE, NULL,
          FAKE, FAKE, FAKE, FAKE, FAKE, ws, NULL]
    a = list(ok); a[22] = ws - 1
    assert L.moe_layer_decode(*a) == -3                     # workspace too small
    a = list(ok); a[20] = NULL
    assert L.moe_layer_decode(*a) == -1                     # out NULL
    a = list(ok); a[5] = 9
    a[22] = L.moe_layer_decode_workspace_bytes(9, k, E, H, I)
    assert L.moe_layer_decode(*a) == -4                     # T > 8
    a = list(ok); a[8] = 9
    a[22] = L.moe_layer_decode_workspace_bytes(T, 9, E, H, I)
    assert L.moe_layer_decode(*a) == -4                     # T * top_k > 64
    a = list(ok); a[12] = R(_tensor(E, H, I, layout=0))
    assert L.moe_layer_decode(*a) == -4                     # canonical layout
    a = list(ok); a[12] = R(_tensor(E, H, I + 64))
    assert L.moe_layer_decode(*a) == -2                     # descriptor shape
    a = list(ok); a[5] = 0
    assert L.moe_layer_decode(*a) == 0                      # T = 0: nothing queued
