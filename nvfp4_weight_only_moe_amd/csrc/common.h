// Device-side helpers shared by the gfx950 kernels of the NVFP4 MoE block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

typedef _Float16 f16;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;
constexpr int kXcds = 8;  // XCDs of the MI355X: workgroup b runs on XCD b % 8

// ---- bf16 <-> f32 (bit patterns) -----------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
// round to nearest even; NaN stays NaN (quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// round to nearest even by the hardware conversion (one instruction; a NaN
// becomes a quiet NaN): for results that are never NaN by construction
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// ---- NVFP4 decode ----------------------------------------------------------
// E2M1 x E4M3 products have at most 6 significant bits and lie in
// [2^-10, 2688]: exact in f16.  So a block decodes as: hardware FP4 -> f16
// conversion of the E2M1 codes (scale operand 1.0), times the E4M3 block scale
// converted to f16 by the hardware FP8 conversion, in one packed f16 multiply.

// Two E4M3 block-scale codes (bits 0..7 and 8..15) -> (s0, s1) in f16, exact.
__device__ __forceinline__ f16x2 block_scales_f16(uint32_t two_codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_codes, 1.0f, false);
}

// 8 E2M1 codes (one dword, element 0 in the low nibble) times block scale s
// -> 8 f16 in MFMA operand order.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16 s) {
  const f16x2 ss = {s, s};
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ---- int4 weight formats --------------------------------------------------
// An E4M3 byte with value 0..15 encodes exactly q * 2^-9 (subnormals m * 2^-9
// for q < 8, exponent 1 for 8 <= q < 16), linear in q.  So masking each code
// into a byte of its own and running the hardware FP8 -> f16 conversion with
// scale 2^9 gives q as an exact f16, two codes per conversion.  Tiled int4
// dwords hold their nibbles in the order this wants: byte b has element b in
// its low nibble and element b + 4 in its high nibble.
__device__ __forceinline__ void int4_codes_f16(uint32_t w, f16x2 &e01, f16x2 &e23, f16x2 &e45,
                                               f16x2 &e67) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  e01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);
  e23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);
  e45 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);
  e67 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);
}
// the tiled nibble order of a canonical dword (element j in bits 4j):
// element j < 4 moves to bits 8j, element j >= 4 to bits 8(j - 4) + 4
__device__ __forceinline__ uint32_t int4_tile_dword(uint32_t c) {
  uint32_t t = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pos = j < 4 ? 8 * j : 8 * (j - 4) + 4;
    t |= ((c >> (4 * j)) & 15u) << pos;
  }
  return t;
}

// Decode of one weight format inside the expert kernels: the bytes of scale
// data a lane loads per 128-K unit (its 32 elements of one row), their
// per-unit preparation, and the 8 f16 operands of dword j of the lane's 16
// packed bytes.
template <int FMT>
struct WeightFmt;
template <>
struct WeightFmt<MOE_FORMAT_NVFP4> {
  static constexpr int kScaleBytes = 2;  // two E4M3 block codes
  struct Prep {
    f16x2 s;
  };
  static __device__ __forceinline__ Prep prep(uint32_t raw) { return {block_scales_f16(raw)}; }
  static __device__ __forceinline__ f16x8 dequant(uint32_t w, const Prep &p, int j) {
    return dequant8(w, p.s[j >> 1]);
  }
};
template <>
struct WeightFmt<MOE_FORMAT_Q4_0> {
  static constexpr int kScaleBytes = 2;  // fp16 d; w = (q - 8) d = fma(q, d, -8d), -8d exact
  struct Prep {
    f16x2 d, nb;
  };
  static __device__ __forceinline__ Prep prep(uint32_t raw) {
    const f16 d = __builtin_bit_cast(f16, (uint16_t)raw);
    const f16 nb = d * (f16)(-8.0f);
    return {f16x2{d, d}, f16x2{nb, nb}};
  }
  static __device__ __forceinline__ f16x8 dequant(uint32_t w, const Prep &p, int) {
    f16x2 a, b, c, d;
    int4_codes_f16(w, a, b, c, d);
    a = __builtin_elementwise_fma(a, p.d, p.nb);
    b = __builtin_elementwise_fma(b, p.d, p.nb);
    c = __builtin_elementwise_fma(c, p.d, p.nb);
    d = __builtin_elementwise_fma(d, p.d, p.nb);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
};
template <>
struct WeightFmt<MOE_FORMAT_AFF4> {
  static constexpr int kScaleBytes = 4;  // fp16 s, fp16 b; w = fma(q, s, b)
  struct Prep {
    f16x2 s, b;
  };
  static __device__ __forceinline__ Prep prep(uint32_t raw) {
    const f16 s = __builtin_bit_cast(f16, (uint16_t)raw);
    const f16 b = __builtin_bit_cast(f16, (uint16_t)(raw >> 16));
    return {f16x2{s, s}, f16x2{b, b}};
  }
  static __device__ __forceinline__ f16x8 dequant(uint32_t w, const Prep &p, int) {
    f16x2 a, b, c, d;
    int4_codes_f16(w, a, b, c, d);
    a = __builtin_elementwise_fma(a, p.s, p.b);
    b = __builtin_elementwise_fma(b, p.s, p.b);
    c = __builtin_elementwise_fma(c, p.s, p.b);
    d = __builtin_elementwise_fma(d, p.s, p.b);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
};

// ---- buffer loads ------------------------------------------------------------
// Raw buffer resource over [base, base + bytes): a load at a byte offset at
// or beyond `bytes` returns zeros (hardware range check), which is how lanes
// past the end of a tensor or tile read zeros without a select.
constexpr uint32_t kOOB = 0x80000000u;  // an offset outside every buffer used here
// `off` (< 2^31) when ok, else an offset past the buffer (the load returns
// zeros), without a branch: a select around a load's address can otherwise be
// compiled into two loads under complementary masks, the second waiting for
// every load in flight (it rewrites the same registers)
__device__ __forceinline__ uint32_t off_if(bool ok, uint32_t off) {
  return off | ((uint32_t)!ok << 31);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// streamed once: non-temporal
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// the scale data of one lane and unit of a weight format
template <int SB>
__device__ __forceinline__ uint32_t load_scale(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return SB == 4 ? bload4(r, off) : bload2(r, off);
}

// C[16x16] += A[16x32] * B[32x16]; lane l holds A[l%16][8(l/16)+i],
// B[8(l/16)+i][l%16] and C[4(l/16)+j][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---- per-row power-of-two rescale to f16 ---------------------------------
// A row whose largest magnitude is M gets the factor 2^(14 - floor(log2 M)),
// putting M in [2^14, 2^15): every bf16 value down to M * 2^-29 converts to
// f16 exactly and nothing overflows.  The returned exponent is what the fp32
// sums are multiplied back by (2^(expo - 14)).  It is clamped at -110, so the
// factor stays finite (at most 2^124) for rows below 2^-110: their values
// then land below the f16 range's top and the smallest underflow to zero.
constexpr int kMinRowExponent = -110;
__device__ __forceinline__ int row_exponent(float amax) {
  if (!(amax > 0.0f) || !(amax < __builtin_huge_valf())) return 0;  // zero / non-finite row
  int e;
  (void)__builtin_frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1)
  return max(e - 1, kMinRowExponent);  // floor(log2 amax), clamped
}

// Maximum over the 16 lanes of each DPP row (lanes 16g .. 16g + 15), in every
// lane of the row: DPP moves (xor 1, xor 2, half-row mirror, row mirror)
// instead of LDS permutes.  Unsigned: non-negative floats compare like their
// bit patterns.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return v;
}
// |b| of a bf16 as the bit pattern of an f32 (ordered like the magnitudes;
// NaN counts as 0)
__device__ __forceinline__ uint32_t bf16_abs_bits(uint16_t b) {
  const uint32_t mag = b & 0x7FFFu;
  return mag > 0x7F80u ? 0u : mag << 16;
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts, then the
// row broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_zero_fill(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_zero_fill<0x111, 0xF>(v);  // row_shr:1
  v += dpp_zero_fill<0x112, 0xF>(v);  // row_shr:2
  v += dpp_zero_fill<0x114, 0xF>(v);  // row_shr:4
  v += dpp_zero_fill<0x118, 0xF>(v);  // row_shr:8 (rows of 16 now scanned)
  v += dpp_zero_fill<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_zero_fill<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- expert-input prep of one token row, by one wave ----------------------
// Row maximum -> exponent -> f16 row scaled by 2^(14 - exponent), row-major
// [T][H], and the exponent.  NORM: the row is first the learned RMSNorm of x,
// y = x / sqrt(mean(x^2) + eps) * norm_w, in fp32 from the bf16 row (sum of
// squares in a fixed order).  A lane keeps its (up to kPrepV) 16-byte pieces
// of the row in registers between the passes, so the row is read once.
constexpr int kPrepV = 8;  // H <= 64 * 8 * kPrepV; longer rows take a second read

template <bool NORM>
__device__ __forceinline__ void prep_row(const uint16_t *__restrict__ x,
                                         const uint16_t *__restrict__ norm_w, float eps, int H,
                                         int t, uint16_t *__restrict__ x16,
                                         int32_t *__restrict__ x_exp) {
  const int lane = threadIdx.x & 63;
  const uint16_t *row = x + (size_t)t * H;
  u32x4 keep[kPrepV], gkeep[kPrepV];
#pragma unroll
  for (int v = 0; v < kPrepV; ++v) {
    const int k = (v * kWave + lane) * 8;
    keep[v] = k < H ? *(const u32x4 *)(row + k) : u32x4{0, 0, 0, 0};
    if (NORM) gkeep[v] = k < H ? *(const u32x4 *)(norm_w + k) : u32x4{0, 0, 0, 0};
  }
  // 1 / rms of the row (NORM)
  float inv = 1.0f;
  if (NORM) {
    float ss = 0.0f;
#pragma unroll
    for (int v = 0; v < kPrepV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(keep[v][i] << 16), hi = __uint_as_float(keep[v][i] & 0xFFFF0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    for (int k = (kPrepV * kWave + lane) * 8; k < H; k += kWave * 8) {  // rows longer than kept
      const u32x4 v = *(const u32x4 *)(row + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
    ss = wave_sum(ss);
    inv = 1.0f / sqrtf(ss / (float)H + eps);
  }
  // the 8 expert-input values of a 16-byte piece (bf16 x, and norm_w when NORM)
  auto values = [&](const u32x4 &xv, const u32x4 &gv, float (&y)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = __uint_as_float(xv[i] << 16);
      y[2 * i + 1] = __uint_as_float(xv[i] & 0xFFFF0000u);
      if (NORM) {
        y[2 * i] = y[2 * i] * inv * __uint_as_float(gv[i] << 16);
        y[2 * i + 1] = y[2 * i + 1] * inv * __uint_as_float(gv[i] & 0xFFFF0000u);
      }
    }
  };
  auto gload = [&](int k) { return NORM ? *(const u32x4 *)(norm_w + k) : u32x4{0, 0, 0, 0}; };
  float amax = 0.0f;
  for (int k = (kPrepV * kWave + lane) * 8; k < H; k += kWave * 8) {
    float y[8];
    values(*(const u32x4 *)(row + k), gload(k), y);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
  }
#pragma unroll
  for (int v = 0; v < kPrepV; ++v) {
    float y[8];
    values(keep[v], gkeep[v], y);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
  }
  amax = wave_max(amax);
  const int ex = row_exponent(amax);
  const float f = __builtin_ldexpf(1.0f, 14 - ex);
  auto convert = [&](const u32x4 &xv, const u32x4 &gv) {
    float y[8];
    values(xv, gv, y);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16 lo = (f16)(y[2 * i] * f);
      const f16 hi = (f16)(y[2 * i + 1] * f);
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return o;
  };
#pragma unroll
  for (int v = 0; v < kPrepV; ++v) {
    const int k = (v * kWave + lane) * 8;
    if (k < H) *(u32x4 *)(x16 + (size_t)t * H + k) = convert(keep[v], gkeep[v]);
  }
  for (int k = (kPrepV * kWave + lane) * 8; k < H; k += kWave * 8)
    *(u32x4 *)(x16 + (size_t)t * H + k) = convert(*(const u32x4 *)(row + k), gload(k));
  if (lane == 0) x_exp[t] = ex;
}

// Router logits of many tokens in moe_route_bucket: 64 tokens x EXP experts
// per workgroup, split along K into ks slices that write partial sums into
// the moe_bucket workspace (the selection kernel adds them in slice order).
// Up to 512 tiles of 32 experts the tiles stay at 32 experts and the split
// brings the grid to about 1024 workgroups; beyond, EXP = kRouteBigExp
// experts per tile (each token row read E / EXP times instead of E / 32) and
// the split restores the grid.  Host side; a function of T and E only, so
// that the workspace size is.  ks = 0: no split (moe_route's kernels).
// (16384 tokens, 128 experts: the routing stage 141 -> 125 us with 128, 128
// with 64; 8192 tokens: unchanged)
constexpr int kRouteBigExp = 128;
inline void route_split_cfg(int T, int E, int *exp, int *ks) {
  const long long tok = (T + 63) / 64;
  *exp = tok * ((E + 31) / 32) >= 512 ? kRouteBigExp : 32;
  const long long tiles = tok * ((E + *exp - 1) / *exp);
  if (T <= 64 || (*exp == 32 && tiles >= 512)) {
    *ks = 0;
    return;
  }
  const long long k = (1024 + tiles - 1) / tiles;
  *ks = k > 8 ? 8 : (int)k;  // at most the selection kernel's kRouteMaxKs
}
inline int route_split_ks(int T, int E) {
  int exp, ks;
  route_split_cfg(T, E, &exp, &ks);
  return ks;
}
// the partial buffers in a moe_bucket workspace: [ks][T][E] and [ks][T]
void route_partials(void *workspace, int T, int top_k, int E, float **part, float **pss);

// The expert-input prep handed to the decode selection kernel
// (moe_route_bucket_prep); x16 == nullptr: none.
struct PrepArgs {
  const uint16_t *x;       // [T][H] bf16 rows (the router's input)
  const uint16_t *norm_w;  // [H] learned RMSNorm weight, or nullptr: the expert input is x
  float norm_eps;
  int H, P;
  uint16_t *x16;           // [T][H] f16 expert input
  int32_t *x_exp;          // [T]
  uint32_t *a_max;         // [P], zeroed
};

// Host: the expert-input buffers of an expert workspace (f16 rows, their
// exponents, the row maxima of A), with the checks of nvfp4_expert_prep.
int expert_prep_buffers(int T, int top_k, int E, int H, int I, void *workspace, size_t ws_bytes,
                        uint16_t **x16, int32_t **x_exp, uint32_t **a_max);

}  // namespace moe

// Host-side helpers.
#include <tuple>
#include <utility>

namespace moe {
// Launch a kernel through hipLaunchKernel so that the status of this launch
// (and not a stale error of an unrelated earlier runtime call) is returned.
template <typename... KArgs, typename... Args, size_t... Is>
hipError_t launch_impl(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                       hipStream_t stream, std::index_sequence<Is...>, Args &&...args) {
  std::tuple<KArgs...> vals(std::forward<Args>(args)...);
  void *ptrs[sizeof...(KArgs) + 1] = {(void *)&std::get<Is>(vals)...};
  return hipLaunchKernel((const void *)kernel, grid, block, ptrs, lds, stream);
}
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                  Args &&...args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  return launch_impl(kernel, grid, block, lds, stream, std::index_sequence_for<KArgs...>{},
                     std::forward<Args>(args)...);
}
}  // namespace moe

#define MOE_LAUNCH(...)                                              \
  do {                                                               \
    if (::moe::launch(__VA_ARGS__) != hipSuccess) return MOE_ERR_LAUNCH; \
  } while (0)

static inline size_t moe_align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
