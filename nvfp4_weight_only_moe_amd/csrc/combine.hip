// moe_combine: weighted sum of a token's routed expert outputs
// ("Gemma 4 26B-A4B (MoE) - Core AI", Architecture: sum over k of w_k h2_k).
// out[t] = sum_j w[t][j] * Y[rank(t, j)], fixed order j = 0, 1, ..., fp32
// accumulation, one bf16 rounding.  Workgroup (t, c) covers token t's columns
// 1024c .. 1024c + 1023; each thread owns 8 consecutive outputs (16-byte
// loads and stores), so even a decode batch spreads over many workgroups.
#include "common.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 128;

__global__ __launch_bounds__(kCombineThreads) void k_combine(const uint16_t *__restrict__ y,
                                                 const float *__restrict__ w,
                                                 const int32_t *__restrict__ rank, int T, int K,
                                                 int H, uint16_t *__restrict__ out) {
  const int t = blockIdx.x;
  const int P = T * K;
  // ranks and weights first, then every row load issued before any is used,
  // so the loads of the K rows overlap instead of queueing one by one
  int rk[MOE_MAX_TOPK];
  float wk[MOE_MAX_TOPK];
  uint32_t valid = 0;  // bit j: slot j has a rank inside [0, P)
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    rk[j] = 0;
    wk[j] = 0.0f;
    if (j < K) {
      const int rr = rank[(size_t)t * K + j];
      if (rr >= 0 && rr < P) {
        rk[j] = rr;
        wk[j] = w[(size_t)t * K + j];
        valid |= 1u << j;
      }
    }
  }
  const int c = (blockIdx.y * kCombineThreads + threadIdx.x) * 8;
  if (c < H) {
    u32x4 v[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if ((valid >> j) & 1u) v[j] = *(const u32x4 *)(y + (size_t)rk[j] * H + c);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if ((valid >> j) & 1u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wk[j], __uint_as_float(v[j][i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wk[j], __uint_as_float(v[j][i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = f32x2_to_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *(u32x4 *)(out + (size_t)t * H + c) = o;
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_combine(const uint16_t *y_sorted, const float *topk_w, const int32_t *pair_rank,
                           int32_t T, int32_t top_k, int32_t H, uint16_t *out, void *stream) {
  using namespace moe;
  if (T > 0 && (!y_sorted || !topk_w || !pair_rank || !out)) return MOE_ERR_NULL;
  if (T < 0 || top_k <= 0 || H <= 0 || H % 8) return MOE_ERR_SHAPE;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  MOE_LAUNCH(k_combine, dim3(T, (H + 8 * kCombineThreads - 1) / (8 * kCombineThreads)),
             dim3(kCombineThreads), 0, (hipStream_t)stream, y_sorted, topk_w, pair_rank, T, top_k,
             H, out);
  return MOE_OK;
}
