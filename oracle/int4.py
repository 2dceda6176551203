"""Two 4-bit integer weight formats for the expert block, in float64 (oracle;
test infrastructure only).

"Gemma 4 26B-A4B (MoE) - Core AI", Compression recipe: that port stores the
routed experts as affine int4 ("aff4"), one fp16 scale and one fp16 bias per
(output row, block of 32 along K); the checkpoint was trained on the ggml q4_0
grid, w = (q - 8) d with one scale d per block of 32 (16 uniform levels), which
an affine block-32 grid represents exactly with scale d and bias -8d.  The
MSE-optimal clip search of that recipe is a quantiser and not part of the
block.

Readings (the page gives the formulas, not the bytes):
* q is an unsigned 4-bit code 0..15; byte j of a row holds element 2j in its
  low nibble and 2j+1 in its high nibble (as for NVFP4).
* aff4: w = q * s + b;  q4_0: w = (q - 8) * d;  s, b, d are IEEE binary16, one
  per (row, block of 32 along K), stored as bit patterns.
* The expert kernels multiply f16 operands: each weight enters the matrix
  cores rounded once to f16 (round to nearest, ties to even).  ``round_f16``
  is that rounding of the exact value.
"""
import numpy as np

GROUP = 32


def f16_bits_to_f64(bits):
    """IEEE binary16 bit patterns -> float64, by the definition: sign, 5-bit
    exponent (bias 15), 10-bit fraction; exponent 0 is subnormal (f * 2^-24),
    exponent 31 is inf (fraction 0) or NaN."""
    b = np.asarray(bits, dtype=np.int64)
    s = np.where((b >> 15) & 1 == 1, -1.0, 1.0)
    e = (b >> 10) & 31
    f = b & 1023
    normal = (1.0 + f / 1024.0) * np.exp2(e - 15.0)
    sub = f * 2.0 ** -24
    val = np.where(e == 0, sub, normal)
    val = np.where(e == 31, np.where(f == 0, np.inf, np.nan), val)
    return s * val


def round_f16(x):
    """Round float64 values to the nearest binary16 value (ties to even;
    beyond the largest finite value, 65504, to +-inf), as float64."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def unpack_codes(packed):
    """[..., K/2] bytes -> [..., K] codes 0..15 (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def decode_q4_0(packed, d_bits):
    """w[n, k] = (q[n, k] - 8) * d[n, k // 32]   (float64, exact)."""
    q = unpack_codes(packed)
    d = f16_bits_to_f64(d_bits)
    return (q - 8) * np.repeat(d, GROUP, axis=-1)


def decode_aff4(packed, sb_bits):
    """w[n, k] = q[n, k] * s[n, k // 32] + b[n, k // 32]   (float64, exact);
    sb_bits [..., K/32, 2] holds (s, b)."""
    q = unpack_codes(packed)
    sb = np.asarray(sb_bits)
    s = np.repeat(f16_bits_to_f64(sb[..., 0]), GROUP, axis=-1)
    b = np.repeat(f16_bits_to_f64(sb[..., 1]), GROUP, axis=-1)
    return q * s + b


def int4_weights(fmt, packed, scales):
    """Callable e -> decoded float64 [N, K] of expert e of a stack."""
    dec = {"q4_0": decode_q4_0, "aff4": decode_aff4}[fmt]

    def get(e):
        return dec(packed[e], scales[e])
    return get
