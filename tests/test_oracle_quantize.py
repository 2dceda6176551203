"""Pins of the oracle's NVFP4 quantiser (CPU only): round-trip idempotence,
error bound, the pages' block-scale formula, grid fixed points, special cases."""
import numpy as np
import pytest

from oracle import formats as F
from oracle.quantize import quantize, global_scale
import moe_synth as S


def _bf16_weights(n, k, seed, std=0.02):
    rng = np.random.default_rng(seed)
    bits = S.f32_to_bf16_bits((rng.standard_normal((n, k)) * std).astype(np.float32))
    return F.bf16_bits_to_f64(bits)


@pytest.mark.parametrize("shape", [(64, 256), (48, 704), (16, 2816)])
def test_roundtrip_idempotent(shape):
    w = _bf16_weights(*shape, seed=shape[0])
    p1, s1, g1 = quantize(w)
    w_hat = F.dequantize(p1, s1, g1)
    p2, s2, g2 = quantize(w_hat)
    assert g1 == g2
    assert np.array_equal(s1, s2)
    assert np.array_equal(p1, p2)


def test_error_bound_and_pages_block_scale():
    w = _bf16_weights(96, 1024, seed=3)
    packed, sc, g = quantize(w)
    s_b = F.e4m3_decode(sc) * g                                  # [N, K/16]
    w_hat = F.dequantize(packed, sc, g)
    err = np.abs(w - w_hat).reshape(96, 64, 16).max(axis=-1)
    assert np.all(err <= s_b + 1e-300)                           # half the widest gap (4..6) or clip
    amax_b = np.abs(w).reshape(96, 64, 16).max(axis=-1)
    # pages: S_block = max|w| / V_max, V_max = 6; E4M3 rounding is within 2^-4 relative
    rel = np.abs(s_b * 6.0 / amax_b - 1.0)
    assert rel.max() <= 2.0 ** -4
    # and the largest block lands on the largest E4M3 value
    assert sc.max() == 0x7E


def test_global_scale_formula():
    w = _bf16_weights(8, 64, seed=5)
    assert global_scale(w) == float(np.float32(np.abs(w).max() / 2688.0))


def test_block_on_grid_quantises_to_itself():
    # g = 1 exactly (max|w| = 2688), every block has a +-6*448 element, so each
    # block scale is 448 and the codes are the E2M1 values themselves
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(4, 64)).astype(np.uint8)
    codes[:, ::16] = 7                                           # a 6.0 in every block
    codes[codes == 8] = 0                                        # no -0 in the input
    w = F.e2m1_decode(codes) * 448.0
    packed, sc, g = quantize(w)
    assert g == 1.0
    assert np.all(sc == 0x7E)
    assert np.array_equal(F.unpack_nibbles(packed), codes)


def test_zero_tensor_and_zero_block():
    z = np.zeros((4, 32))
    packed, sc, g = quantize(z)
    assert g == 0.0 and not packed.any() and not sc.any()
    w = _bf16_weights(4, 32, seed=9)
    w[:, 16:] = 0.0
    packed, sc, g = quantize(w)
    assert np.all(sc[:, 1] == 0)
    assert not F.unpack_nibbles(packed)[:, 16:].any()


def test_negative_values_sign_and_symmetry():
    w = _bf16_weights(16, 128, seed=11)
    p1, s1, g1 = quantize(w)
    p2, s2, g2 = quantize(-w)
    c1, c2 = F.unpack_nibbles(p1), F.unpack_nibbles(p2)
    assert g1 == g2 and np.array_equal(s1, s2)
    nz = (c1 & 7) != 0
    assert np.array_equal(c1[nz] ^ 8, c2[nz])
    assert np.array_equal(c1[~nz], c2[~nz])
