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

// ---- NVFP4 block-scale decode --------------------------------------------
// An E4M3 block scale s is split as s = 2^E * m with m in [1, 2) (sign on m):
// the power of two rides in the hardware FP4 conversion (which uses only the
// exponent of its f32 scale operand), m is applied with one packed f16
// multiply.  E2M1 x 2^E and its product with m are exact in f16.
struct BlockScale {
  float pow2;   // 2^E as f32 (exponent bits only); 0 for a zero scale
  f16x2 mant;   // (m, m) as f16
};

__device__ __forceinline__ BlockScale decode_block_scale(uint32_t code) {
  float s = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);  // OCP E4M3 -> f32, exact
  uint32_t b = __float_as_uint(s);
  BlockScale r;
  r.pow2 = __uint_as_float(b & 0x7F800000u);
  uint16_t m16 = (uint16_t)(((b >> 16) & 0x8000u) | 0x3C00u | ((b & 0x007FFFFFu) >> 13));
  f16 m = __builtin_bit_cast(f16, m16);
  r.mant = f16x2{m, m};
  return r;
}

// 8 E2M1 codes (one dword, element 0 in the low nibble) times a block scale
// -> 8 f16 in MFMA operand order.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, const BlockScale &s) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 0);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 1);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 2);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 3);
  a *= s.mant;
  b *= s.mant;
  c *= s.mant;
  d *= s.mant;
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
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
// sums are multiplied back by (2^(expo - 14)).
__device__ __forceinline__ int row_exponent(float amax) {
  if (!(amax > 0.0f) || !(amax < __builtin_huge_valf())) return 0;  // zero / non-finite row
  int e;
  (void)__builtin_frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1)
  return e - 1;                      // floor(log2 amax)
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
