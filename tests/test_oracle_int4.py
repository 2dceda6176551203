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


def test_synthetic_int4_stacks_follow_their_recipe():
    """The seeded int4 inputs: deterministic per (format, layer, projection,
    expert), stored shapes, fp16 scales inside the drawn ranges, and decoded
    weights of the size of the bf16 N(0, 0.02) weights."""
    import moe_synth as S
    for fmt in ("q4_0", "aff4"):
        p, s = S.int4_expert(fmt, 0, S.GATE, 5)
        p2, s2 = S.int4_expert(fmt, 0, S.GATE, 5)
        assert np.array_equal(p, p2) and np.array_equal(s, s2)
        assert not np.array_equal(p, S.int4_expert(fmt, 0, S.GATE, 6)[0])
        assert p.shape == (S.I, S.H // 2) and p.dtype == np.uint8
        assert s.shape == (S.I, S.H // 32 * S.INT4_SCALE_BYTES[fmt])
        bits = s.view(np.uint16)
        if fmt == "q4_0":
            d = Q.f16_bits_to_f64(bits)
            assert d.min() >= 0.004 - 1e-5 and d.max() <= 0.008 + 1e-5
            w = Q.decode_q4_0(p, bits)
        else:
            sb = Q.f16_bits_to_f64(bits.reshape(S.I, -1, 2))
            assert sb[..., 0].min() >= 0.004 - 1e-5 and sb[..., 0].max() <= 0.008 + 1e-5
            assert sb[..., 1].min() >= -0.06 - 1e-4 and sb[..., 1].max() <= -0.035 + 1e-4
            w = Q.decode_aff4(p, bits.reshape(S.I, -1, 2))
        assert 0.015 < w.std() < 0.045
        # every code appears, with roughly uniform frequency
        cnt = np.bincount(Q.unpack_codes(p).ravel(), minlength=16)
        assert cnt.min() > 0.9 * cnt.mean()
    c = S.small_int4_case(3, "aff4", 5, 128, 64, 8, 2)
    assert c["gate"][0].shape == (8, 64, 64) and c["down"][1].shape == (8, 128, 64 // 32 * 4)
