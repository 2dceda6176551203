// Weight preparation and checks: the NVFP4 block quantiser and the bf16
// decode of one expert tensor, plus the status strings.
//
// Quantiser: "Gemma-4-26B-A4B-it-NVFP4" README, block-quantisation formulas:
// S_block = max|w| / 6 over 16 contiguous inner-dimension elements,
// q = clip(round(w / S_block), -6, 6), here in the two-level form (E4M3 block
// scale x FP32 tensor scale, "Gemma-4-26B-A4B-NVFP4-mlx", Quantization recipe):
//   g    = fl32(max|W| / (6 * 448))                  per expert tensor
//   code = E4M3_rne_sat(amax_block / (6 g))          in IEEE double
//   q    = E2M1_rne(clip(w / (E4M3(code) g), -6, 6)) in IEEE double
// Three kernels: per-expert max|W| (integer atomicMax of float bits, one per
// workgroup: exact and order-independent), the per-block quantisation, and
// the write of g.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t *__restrict__ p, int n, uint32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// max|W| of expert blockIdx.y: each workgroup takes a contiguous slice,
// reduces it in registers and LDS, and issues one integer atomicMax of the
// float bits (gridDim.x atomics per expert: same-address atomics serialise,
// so there are few of them).
__global__ __launch_bounds__(256) void k_absmax(const uint16_t *__restrict__ w, size_t per_e,
                                                uint32_t *__restrict__ amax_bits) {
  __shared__ float s_m[4];
  const int e = blockIdx.y;
  const uint16_t *base = w + (size_t)e * per_e;
  const size_t n8 = per_e / 8;  // 16-byte pieces (K % 32 == 0)
  const size_t b0 = n8 * blockIdx.x / gridDim.x, b1 = n8 * (blockIdx.x + 1) / gridDim.x;
  float m = 0.0f;
  for (size_t i = b0 + threadIdx.x; i < b1; i += 256) {
    const u32x4 v = *(const u32x4 *)(base + i * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m = fmaxf(m, fabsf(__uint_as_float(v[q] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(v[q] & 0xFFFF0000u)));
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(&amax_bits[e], __float_as_uint(fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]))));
}

// nearest E4M3 code of r >= 0 (ties to even mantissa, saturate at 448)
__device__ uint32_t e4m3_rne_sat(double r) {
  if (!(r < 448.0)) return 0x7E;
  if (r < 0.015625) {                        // below 2^-6: subnormal step 2^-9
    return (uint32_t)rint(r * 512.0);          // 0..8; 8 is code 0x08 = 2^-6
  }
  int ex;
  (void)frexp(r, &ex);                         // r = f 2^ex, f in [0.5, 1)
  int E = ex - 1;                              // floor(log2 r), -6 .. 8
  double q = rint(ldexp(r, 3 - E));            // 8 .. 16
  if (q == 16.0) {
    q = 8.0;
    E += 1;
  }
  return (uint32_t)(((E + 7) << 3) | ((int)q - 8));
}

__device__ double e4m3_value(uint32_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

// nearest E2M1 magnitude code of a in [0, 6], ties to the even code
__device__ uint32_t e2m1_rne(double a) {
  return (uint32_t)(a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) +
         (a > 5.0);
}

__global__ __launch_bounds__(256) void k_quant(const uint16_t *__restrict__ w, int N, int K,
                                               const uint32_t *__restrict__ amax_bits,
                                               uint8_t *__restrict__ packed,
                                               uint8_t *__restrict__ scales) {
  const int e = blockIdx.y;
  const int nb = K / 16;
  const size_t blk = (size_t)blockIdx.x * 256 + threadIdx.x;  // block index within expert
  if (blk >= (size_t)N * nb) return;
  const float g = (float)((double)__uint_as_float(amax_bits[e]) / 2688.0);
  const size_t eoff = (size_t)e * N * K;
  const uint16_t *src = w + eoff + blk * 16;
  float v[16];
  const u32x4 a = *(const u32x4 *)src, b = *(const u32x4 *)(src + 8);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(a[q] << 16);
    v[2 * q + 1] = __uint_as_float(a[q] & 0xFFFF0000u);
    v[8 + 2 * q] = __uint_as_float(b[q] << 16);
    v[8 + 2 * q + 1] = __uint_as_float(b[q] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t code = 0;
  double sb = 0.0;
  if (g > 0.0f) {
    code = e4m3_rne_sat((double)amax / (6.0 * (double)g));
    sb = e4m3_value(code) * (double)g;
  }
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t c = 0;
    if (sb > 0.0) {
      double q = (double)v[i] / sb;
      q = fmin(6.0, fmax(-6.0, q));
      const uint32_t mag = e2m1_rne(fabs(q));
      c = mag | ((q < 0.0 && mag != 0) ? 8u : 0u);
    }
    if (i < 8) lo |= c << (4 * i);
    else hi |= c << (4 * (i - 8));
  }
  *(u32x2 *)(packed + (size_t)e * N * (K / 2) + blk * 8) = u32x2{lo, hi};
  scales[(size_t)e * N * nb + blk] = (uint8_t)code;
}

__global__ void k_write_global(const uint32_t *__restrict__ amax_bits, int E,
                               float *__restrict__ global) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < E) global[e] = (float)((double)__uint_as_float(amax_bits[e]) / 2688.0);
}

// Byte offsets of element (n, k) (k % 8 == 0) of one expert tensor in the
// tiled layout: its packed dword and the first byte of its lane's scale data
// (SB bytes per lane and unit).  Lane l = 16 g + r of unit u of row tile t
// holds row 16t + r, k = 128u + 32g .. +31.
__device__ __forceinline__ void tiled_offsets(size_t n, size_t k, int K, int SB, size_t *pw,
                                              size_t *ps) {
  const size_t t = n / 16, r = n % 16, u = k / 128, g = (k % 128) / 32, w = (k % 32) / 8;
  const size_t lane = 16 * g + r;
  *pw = t * 16 * (size_t)(K / 2) + u * 1024 + lane * 16 + w * 4;
  *ps = t * (size_t)K * SB / 2 + u * 64 * SB + lane * SB;
}
// the canonical offset of the lane scale data of element (n, k): NVFP4 the
// two block codes of k's 32 elements, int4 the fp16 d or (s, b) of k's block
template <int FMT>
__device__ __forceinline__ size_t canonical_scale_offset(size_t n, size_t k, int K) {
  constexpr int SB = WeightFmt<FMT>::kScaleBytes;
  return FMT == MOE_FORMAT_NVFP4 ? n * (K / 16) + (k / 32) * 2 : (n * (K / 32) + k / 32) * SB;
}

// canonical -> tiled, one thread per 16-byte lane slot (int4 formats: the
// nibbles of each dword in the tiled order)
template <int FMT>
__global__ __launch_bounds__(256) void k_repack(const uint8_t *__restrict__ packed,
                                                const uint8_t *__restrict__ scales, int N, int K,
                                                size_t nslots, uint8_t *__restrict__ tp,
                                                uint8_t *__restrict__ ts) {
  constexpr int SB = WeightFmt<FMT>::kScaleBytes;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // (expert, row, 32-k slice)
  if (i >= nslots) return;
  const size_t per_e = (size_t)N * (K / 32);
  const size_t e = i / per_e, rem = i % per_e;
  const size_t n = rem / (K / 32), k = (rem % (K / 32)) * 32;
  size_t pw, ps;
  tiled_offsets(n, k, K, SB, &pw, &ps);
  const uint8_t *src = packed + e * N * (K / 2) + n * (K / 2) + k / 2;
  u32x4 v = *(const u32x4 *)src;
  if (FMT != MOE_FORMAT_NVFP4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = int4_tile_dword(v[q]);
  }
  *(u32x4 *)(tp + e * N * (K / 2) + pw) = v;
  const size_t sbytes = (size_t)N * K * SB / 32;  // per expert
  const uint8_t *ssrc = scales + e * sbytes + canonical_scale_offset<FMT>(n, k, K);
  uint8_t *sdst = ts + e * sbytes + ps;
#pragma unroll
  for (int b = 0; b < SB; ++b) sdst[b] = ssrc[b];
}

// one thread per 8 elements: the expert kernels' decode (WeightFmt), as f16
// bit patterns; BF16: NVFP4 only, widened to bf16 (exact)
template <int FMT, bool BF16>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t *__restrict__ packed,
                                                 const uint8_t *__restrict__ scales, int N, int K,
                                                 int tiled, uint16_t *__restrict__ out) {
  constexpr int SB = WeightFmt<FMT>::kScaleBytes;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // dword index
  if (i >= (size_t)N * K / 8) return;
  const size_t n = i / (K / 8), k = (i % (K / 8)) * 8;
  size_t pw = n * (K / 2) + k / 2, ps = canonical_scale_offset<FMT>(n, k, K);
  if (tiled) tiled_offsets(n, k, K, SB, &pw, &ps);
  uint32_t wv = *(const uint32_t *)(packed + pw);
  if (FMT != MOE_FORMAT_NVFP4 && !tiled) wv = int4_tile_dword(wv);
  uint32_t raw = scales[ps] | ((uint32_t)scales[ps + 1] << 8);
  if (SB == 4) raw |= ((uint32_t)scales[ps + 2] << 16) | ((uint32_t)scales[ps + 3] << 24);
  const f16x8 h = WeightFmt<FMT>::dequant(wv, WeightFmt<FMT>::prep(raw), (int)((k % 32) / 8));
  // f16: the vector's bytes as they are (a bit_cast of a single vector
  // element h[i] would read element 0 with this compiler, so the whole
  // vector is cast)
  u32x4 o = __builtin_bit_cast(u32x4, h);
  if (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = (uint32_t)f32_to_bf16((float)h[2 * q]) | ((uint32_t)f32_to_bf16((float)h[2 * q + 1]) << 16);
  }
  *(u32x4 *)(out + n * K + k) = o;
}

}  // namespace
}  // namespace moe

extern "C" int nvfp4_quantize(const uint16_t *w, int32_t E, int32_t N, int32_t K, uint8_t *packed,
                              uint8_t *scales, float *global, void *stream) {
  using namespace moe;
  if (!w || !packed || !scales || !global) return MOE_ERR_NULL;
  if (E <= 0 || N <= 0 || K <= 0 || K % 32) return MOE_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  // the float output doubles as the per-expert max|W| (float bits) until the end
  uint32_t *amax = (uint32_t *)global;
  MOE_LAUNCH(k_fill_u32, dim3((E + 255) / 256), dim3(256), 0, s, amax, E, 0u);
  const size_t per_e = (size_t)N * K;
  // slices of at least 16 KiB, at most 64 workgroups per expert
  const size_t gx0 = (per_e * 2 + 16383) / 16384;
  const int gx = (int)(gx0 < 64 ? gx0 : 64);
  MOE_LAUNCH(k_absmax, dim3(gx, E), dim3(256), 0, s, w, per_e, amax);
  const size_t nblk = (size_t)N * (K / 16);
  MOE_LAUNCH(k_quant, dim3((unsigned)((nblk + 255) / 256), E), dim3(256), 0, s, w, N, K,
                     amax, packed, scales);
  MOE_LAUNCH(k_write_global, dim3((E + 255) / 256), dim3(256), 0, s, amax, E, global);
  return MOE_OK;
}

extern "C" int nvfp4_repack(const nvfp4_tensor *src, uint8_t *packed_tiled, uint8_t *scales_tiled,
                            void *stream) {
  using namespace moe;
  if (!src || !src->packed || !src->scales || !packed_tiled || !scales_tiled) return MOE_ERR_NULL;
  if (src->E <= 0 || src->N <= 0 || src->N % 16 || src->K <= 0 || src->K % 32) return MOE_ERR_SHAPE;
  if (src->layout != MOE_LAYOUT_CANONICAL) return MOE_ERR_UNSUPPORTED;
  const size_t nslots = (size_t)src->E * src->N * (src->K / 32);
  const dim3 grid((unsigned)((nslots + 255) / 256));
  hipStream_t s = (hipStream_t)stream;
  switch (src->format) {
    case MOE_FORMAT_NVFP4:
      MOE_LAUNCH(k_repack<MOE_FORMAT_NVFP4>, grid, dim3(256), 0, s, src->packed, src->scales,
                 src->N, src->K, nslots, packed_tiled, scales_tiled);
      break;
    case MOE_FORMAT_Q4_0:
      MOE_LAUNCH(k_repack<MOE_FORMAT_Q4_0>, grid, dim3(256), 0, s, src->packed, src->scales,
                 src->N, src->K, nslots, packed_tiled, scales_tiled);
      break;
    case MOE_FORMAT_AFF4:
      MOE_LAUNCH(k_repack<MOE_FORMAT_AFF4>, grid, dim3(256), 0, s, src->packed, src->scales,
                 src->N, src->K, nslots, packed_tiled, scales_tiled);
      break;
    default: return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

namespace {
int dequant_checked(const nvfp4_tensor *w, int32_t e, uint16_t *out, bool bf16, void *stream) {
  using namespace moe;
  if (!w || !out || !w->packed || !w->scales) return MOE_ERR_NULL;
  if (w->N <= 0 || w->K <= 0 || w->K % 32 || e < 0 || e >= w->E) return MOE_ERR_SHAPE;
  if (w->layout != MOE_LAYOUT_CANONICAL && w->layout != MOE_LAYOUT_TILED) return MOE_ERR_UNSUPPORTED;
  if (w->format < MOE_FORMAT_NVFP4 || w->format > MOE_FORMAT_AFF4) return MOE_ERR_UNSUPPORTED;
  if (bf16 && w->format != MOE_FORMAT_NVFP4) return MOE_ERR_UNSUPPORTED;
  if (w->layout == MOE_LAYOUT_TILED && w->N % 16) return MOE_ERR_SHAPE;
  const size_t n8 = (size_t)w->N * w->K / 8;
  const int sb = w->format == MOE_FORMAT_AFF4 ? 4 : 2;
  const uint8_t *p = w->packed + (size_t)e * w->N * (w->K / 2);
  const uint8_t *sc = w->scales + (size_t)e * w->N * w->K * sb / 32;
  const dim3 grid((unsigned)((n8 + 255) / 256));
  hipStream_t s = (hipStream_t)stream;
  const int tiled = w->layout == MOE_LAYOUT_TILED;
  if (bf16) {
    MOE_LAUNCH((k_dequant<MOE_FORMAT_NVFP4, true>), grid, dim3(256), 0, s, p, sc, w->N, w->K, tiled, out);
  } else if (w->format == MOE_FORMAT_NVFP4) {
    MOE_LAUNCH((k_dequant<MOE_FORMAT_NVFP4, false>), grid, dim3(256), 0, s, p, sc, w->N, w->K, tiled, out);
  } else if (w->format == MOE_FORMAT_Q4_0) {
    MOE_LAUNCH((k_dequant<MOE_FORMAT_Q4_0, false>), grid, dim3(256), 0, s, p, sc, w->N, w->K, tiled, out);
  } else {
    MOE_LAUNCH((k_dequant<MOE_FORMAT_AFF4, false>), grid, dim3(256), 0, s, p, sc, w->N, w->K, tiled, out);
  }
  return MOE_OK;
}
}  // namespace

extern "C" int nvfp4_dequant_bf16(const nvfp4_tensor *w, int32_t e, uint16_t *out, void *stream) {
  return dequant_checked(w, e, out, true, stream);
}

extern "C" int moe_dequant_f16(const nvfp4_tensor *w, int32_t e, uint16_t *out, void *stream) {
  return dequant_checked(w, e, out, false, stream);
}

extern "C" const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_WORKSPACE: return "workspace NULL or smaller than required";
    case MOE_ERR_UNSUPPORTED: return "shape not supported by this library";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int moe_abi_version(void) { return (3 << 16) | 0; }
