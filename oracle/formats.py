"""Number formats of NVFP4 in float64 (oracle; test infrastructure only).

NVFP4 as the model cards describe it: 4-bit E2M1 elements, contiguous groups of
16 along the input (inner) dimension, one FP8 E4M3 scale per group and one FP32
scale per tensor ("Gemma-4-26B-A4B-NVFP4-mlx", Quantization recipe table and
Notes; "gemma-4-26B-A4B - NVFP4A16", Quantization details; the largest E2M1
magnitude V_max = 6 from the "Gemma-4-26B-A4B-it-NVFP4" README).

Readings taken where the pages are silent:
* E2M1 magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code bit 3 is the sign.
* E4M3 is the OCP "fn" variant: bias 7, no infinities, S.1111.111 is NaN,
  largest finite 448.
* Packing: byte j of a row holds element 2j in its low nibble and element 2j+1
  in its high nibble; a zero magnitude is always stored as code 0 (no -0).
"""
import numpy as np

# The eight non-negative E2M1 magnitudes, indexed by the 3 low code bits.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e2m1_decode(codes):
    """E2M1 codes (0..15) -> float64: (-1)^bit3 * MAGNITUDES[bits 0..2]."""
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e4m3_decode(codes):
    """OCP E4M3 (fn) byte codes -> float64, all 256 codes.

    b = S EEEE MMM;  E = 0: (-1)^S * M * 2^-9;  E = 15, M = 7: NaN;
    otherwise (-1)^S * (1 + M/8) * 2^(E-7).
    """
    c = np.asarray(codes, dtype=np.int64)
    s = np.where((c >> 7) & 1 == 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    subnormal = m * 2.0 ** -9
    val = s * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def _nearest_code(values, table):
    """Index of the nearest entry of ``table`` (ascending, non-negative) for each
    non-negative value; an exact midpoint goes to the even index.  Brute force
    over every table entry."""
    v = np.asarray(values, dtype=np.float64)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    chunk = 1 << 16
    for s in range(0, flat.size, chunk):
        x = flat[s:s + chunk, None]
        d = np.abs(x - table[None, :])
        best = d.min(axis=1, keepdims=True)
        is_best = d == best
        # candidates: at most two (a tie); prefer the even index
        idx = np.arange(table.size)[None, :]
        even_best = is_best & (idx % 2 == 0)
        pick_even = even_best.any(axis=1)
        first_best = is_best.argmax(axis=1)
        first_even = even_best.argmax(axis=1)
        out[s:s + chunk] = np.where(pick_even, first_even, first_best)
    return out.reshape(v.shape)


# Non-negative finite E4M3 values, codes 0x00..0x7E, ascending with the code.
_E4M3_POS = e4m3_decode(np.arange(0x7F))


def e4m3_encode(r):
    """Non-negative float64 -> E4M3 code, round to nearest, ties to the even
    code (mantissa LSB 0), saturating at 448 (code 0x7E)."""
    r = np.asarray(r, dtype=np.float64)
    if np.any(r < 0) or np.any(np.isnan(r)):
        raise ValueError("e4m3_encode takes non-negative finite values")
    return _nearest_code(np.minimum(r, E4M3_MAX), _E4M3_POS).astype(np.uint8)


def e2m1_encode(v):
    """float64 in [-6, 6] -> E2M1 code, magnitude rounded to the nearest of the
    eight magnitudes, ties to the even code; a zero magnitude gets code 0."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E2M1_MAX):
        raise ValueError("e2m1_encode takes values already clipped to [-6, 6]")
    mag = _nearest_code(np.abs(v), E2M1_MAGNITUDES)
    sign = np.where((v < 0) & (mag != 0), 8, 0)
    return (mag | sign).astype(np.uint8)


def pack_nibbles(codes):
    """[..., K] codes (0..15), K even -> [..., K/2] bytes, low nibble = even k."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("K must be even")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[..., K/2] bytes -> [..., K] codes, inverse of ``pack_nibbles``."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequantize(packed, scale_codes, global_scale, group=16):
    """Two-level NVFP4 decode of one tensor [N, K]:
    ŵ[n,k] = E2M1(code[n,k]) * E4M3(scale[n, k // 16]) * g   (float64)."""
    codes = unpack_nibbles(packed)
    vals = e2m1_decode(codes)
    scales = e4m3_decode(scale_codes)
    return vals * np.repeat(scales, group, axis=-1) * float(global_scale)


def dequantize_no_global(packed, scale_codes, group=16):
    """E2M1 * E4M3 only (the per-tensor FP32 factor left out); every such
    product is exactly representable in bf16 and in f16."""
    codes = unpack_nibbles(packed)
    return e2m1_decode(codes) * np.repeat(e4m3_decode(scale_codes), group, axis=-1)
