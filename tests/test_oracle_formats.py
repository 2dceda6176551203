"""Pins of the oracle's number formats against closed forms, torch's float8
routines and the golden E2M1 rounding table (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_closed_form(code):
    """Value of a 4-bit E2M1 code from its fields: 1 sign bit, 2 exponent bits
    with bias 1, 1 mantissa bit; exponent 0 is subnormal (m * 0.5)."""
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    return s * (m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))


def test_e2m1_decode_matches_bitfield_closed_form():
    for c in range(16):
        assert F.e2m1_decode(c) == _e2m1_closed_form(c), c


def test_e2m1_vmax_is_six():
    # V_max = 6 is the largest E2M1 magnitude (block-quantisation formulas).
    assert F.e2m1_decode(np.arange(16)).max() == 6.0
    assert F.E2M1_MAX == 6.0


def test_e4m3_decode_all_256_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.nanmax(ours) == 448.0
    assert set(np.nonzero(np.isnan(ours))[0].tolist()) == {0x7F, 0xFF}


def test_e4m3_encode_vs_torch_cast_on_midpoints_and_random():
    pos = F.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2.0
    rng = np.random.default_rng(1)
    rand = np.concatenate([rng.uniform(0, 448, 20000), np.exp2(rng.uniform(-12, 8.8, 20000))])
    vals = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), rand])
    vals = vals[(vals >= 0) & (vals <= 448)].astype(np.float32)   # exactly representable inputs
    ours = F.e4m3_encode(vals.astype(np.float64))
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (vals[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_saturates():
    assert F.e4m3_encode(np.array([448.0, 460.0, 1e6])).tolist() == [0x7E, 0x7E, 0x7E]


def test_e2m1_encode_golden_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_rounding.txt"))
            if l.strip() and not l.startswith("#")]
    vals = np.array([float(r[0]) for r in rows])
    codes = np.array([int(r[1]) for r in rows])
    expect = np.array([float(r[2]) for r in rows])
    got = F.e2m1_encode(vals)
    assert got.tolist() == codes.tolist()
    assert np.array_equal(F.e2m1_decode(got), expect)


def test_e2m1_encode_is_nearest_with_even_ties_dense_grid():
    # property check: chosen magnitude is a nearest one; on an exact tie its
    # mantissa bit (code bit 0) is 0
    v = np.linspace(-6, 6, 24001)
    c = F.e2m1_encode(v)
    mags = F.E2M1_MAGNITUDES
    d = np.abs(np.abs(v)[:, None] - mags[None, :])
    best = d.min(axis=1)
    chosen = np.abs(np.abs(v) - np.abs(F.e2m1_decode(c)))
    assert np.array_equal(chosen, best)
    ties = (d == best[:, None]).sum(axis=1) > 1
    assert np.all((c[ties] & 1) == 0)
    assert not np.any(c == 8)  # no negative zero


def test_pack_nibble_order_and_roundtrip():
    assert F.pack_nibbles(np.array([1, 2], np.uint8)).tolist() == [0x21]
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(7, 64)).astype(np.uint8)
    packed = F.pack_nibbles(codes)
    assert packed.shape == (7, 32)
    assert np.array_equal(F.unpack_nibbles(packed), codes)


def test_dequantize_hand_example():
    # one row, two blocks of 16: codes 0..15 in block 0, 7 (=6.0) in block 1;
    # scale codes 0x38 (1.0) and 0x3C (1.5); g = 0.25
    codes = np.concatenate([np.arange(16), np.full(16, 7)]).astype(np.uint8)[None, :]
    packed = F.pack_nibbles(codes)
    sc = np.array([[0x38, 0x3C]], np.uint8)
    w = F.dequantize(packed, sc, 0.25)
    expect0 = np.array([_e2m1_closed_form(c) for c in range(16)]) * 1.0 * 0.25
    assert np.array_equal(w[0, :16], expect0)
    assert np.all(w[0, 16:] == 6.0 * 1.5 * 0.25)


def test_products_exact_in_bf16_and_f16():
    # every E2M1 x E4M3 product (finite codes) is representable in bf16 and f16
    e2 = F.e2m1_decode(np.arange(16))
    e4 = F.e4m3_decode(np.arange(256))
    prod = (e2[:, None] * e4[None, :]).reshape(-1)
    prod = prod[~np.isnan(prod)]
    t = torch.from_numpy(prod)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)
    assert torch.equal(t.to(torch.float16).to(torch.float64), t)


def test_dequantize_no_global_hand_computed():
    """E2M1 x E4M3 with the group of 16 along K ("Gemma-4-26B-A4B-NVFP4-mlx",
    Notes), values worked by hand.  Row 0: codes k % 16, block scales 1.0
    (0x38) and 2.0 (0x40); row 1: the same codes, scales 0.5 (0x30) and 0."""
    codes = np.tile(np.arange(32) % 16, (2, 1)).astype(np.uint8)
    packed = F.pack_nibbles(codes)
    assert packed[0, 0] == 0x10 and packed[0, 7] == 0xFE   # low nibble = even k
    scales = np.array([[0x38, 0x40], [0x30, 0x00]], dtype=np.uint8)
    d = F.dequantize_no_global(packed, scales)
    assert d.shape == (2, 32)
    hand = {(0, 0): 0.0, (0, 1): 0.5, (0, 7): 6.0, (0, 9): -0.5, (0, 15): -6.0,
            (0, 17): 1.0, (0, 23): 12.0, (0, 29): -6.0, (1, 5): 1.5, (1, 7): 3.0,
            (1, 9): -0.25, (1, 14): -2.0, (1, 16): 0.0, (1, 23): 0.0}
    for (n, k), v in hand.items():
        assert d[n, k] == v, (n, k, d[n, k], v)
    # with the tensor scale: the same products times g (same multiplication order)
    g = 0.0078125 * 3
    assert np.array_equal(F.dequantize(packed, scales, g), d * g)


def test_dequantize_no_global_times_g_is_dequantize():
    rng = np.random.default_rng(9)
    packed = rng.integers(0, 256, (8, 64), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (8, 8), dtype=np.uint8)
    g = float(np.float32(0.0123))
    assert np.array_equal(F.dequantize_no_global(packed, scales) * g, F.dequantize(packed, scales, g))
