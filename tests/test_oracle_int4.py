"""Pins of the oracle's int4 weight formats (q4_0, aff4): the binary16 decode
against numpy's float16 for every bit pattern, closed forms of both grids, the
block-of-32 structure, q4_0 as the aff4 special case the Core AI page states
(scale d, bias -8d), and the f16 rounding."""
import numpy as np

from oracle import int4 as Q


def test_f16_decode_every_pattern_vs_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    got = Q.f16_bits_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~both_nan], ref[~both_nan])


def _f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def test_q4_0_closed_forms():
    d = 0.015625                                   # 2^-6
    codes = np.arange(16)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)      # k = 0..15
    row = np.concatenate([packed, np.zeros(8, np.uint8)])             # K = 32
    w = Q.decode_q4_0(row[None], _f16([[d]]))[0]
    assert np.array_equal(w[:16], (codes - 8) * d)                    # 16 uniform levels
    assert w[8] == 0.0 and w[0] == -8 * d and w[15] == 7 * d
    assert np.all(w[16:] == -8 * d)                                   # code 0


def test_aff4_closed_forms_and_blocks():
    s, b = 0.25, -1.5
    packed = np.full((1, 32), 0xF0, np.uint8)                         # K = 64: q = 0, 15, 0, 15 ...
    sb = np.array([[[s, b], [0.0, 0.0]]])                             # block 1 all zero
    w = Q.decode_aff4(packed, _f16(sb).reshape(1, 2, 2))[0]
    assert np.array_equal(w[:32:2], np.full(16, b))
    assert np.array_equal(w[1:32:2], np.full(16, 15 * s + b))
    assert np.all(w[32:] == 0.0)


def test_q4_0_is_aff4_with_bias_minus_8d():
    rng = np.random.default_rng(1)
    packed = rng.integers(0, 256, (3, 64), dtype=np.uint8)           # K = 128
    d = rng.uniform(1e-3, 1e-2, (3, 4)).astype(np.float16)
    sb = np.stack([d, (-8 * d.astype(np.float64)).astype(np.float16)], axis=-1)   # -8d exact
    assert np.array_equal(Q.decode_q4_0(packed, d.view(np.uint16)),
                          Q.decode_aff4(packed, sb.view(np.uint16)))


def test_round_f16_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -10
    assert Q.round_f16(one + ulp / 2) == one                          # tie -> even (1.0)
    assert Q.round_f16(one + 1.5 * ulp) == one + 2 * ulp              # tie -> even
    assert Q.round_f16(one + 0.51 * ulp) == one + ulp
    assert Q.round_f16(65520.0) == np.inf and Q.round_f16(65519.0) == 65504.0
    x = np.random.default_rng(2).standard_normal(1000)
    r = Q.round_f16(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -11 + 2.0 ** -25)
