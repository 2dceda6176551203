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

// The combine followed by the learned RMSNorm of the summed row ("Gemma 4
// 26B-A4B (MoE) - Core AI", Architecture sketch: post_feedforward_layernorm_2
// of the weighted sum, then the residual add and layer_scalar):
//   s = sum_j w[t][j] * Y[rank(t, j)]            (fp32, order j = 0, 1, ...)
//   out[t] = (residual[t] + s / sqrt(mean(s^2) + eps) * norm_w) * layer_scalar
// rounded once to bf16.  One workgroup per token (the norm needs the whole
// row): thread i owns columns 8(i + 256 q), q < kNormPieces, kept in
// registers between the sum of squares and the output.
constexpr int kNormThreads = 256;
constexpr int kNormPieces = 4;  // H <= 8 * 256 * 4 = 8192

__global__ __launch_bounds__(kNormThreads) void k_combine_rmsnorm(
    const uint16_t *__restrict__ y, const float *__restrict__ w, const int32_t *__restrict__ rank,
    const uint16_t *__restrict__ norm_w, float eps, const uint16_t *residual, float layer_scalar,
    int T, int K, int H, uint16_t *out) {
  __shared__ float s_ss[kNormThreads / kWave];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int P = T * K;
  int rk[MOE_MAX_TOPK];
  float wk[MOE_MAX_TOPK];
  uint32_t valid = 0;
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
  float acc[kNormPieces][8];
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < kNormPieces; ++q) {
    const int c = (q * kNormThreads + tid) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[q][i] = 0.0f;
    if (c < H) {
      u32x4 v[MOE_MAX_TOPK];
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j)
        if ((valid >> j) & 1u) v[j] = *(const u32x4 *)(y + (size_t)rk[j] * H + c);
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if ((valid >> j) & 1u) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[q][2 * i] = fmaf(wk[j], __uint_as_float(v[j][i] << 16), acc[q][2 * i]);
            acc[q][2 * i + 1] = fmaf(wk[j], __uint_as_float(v[j][i] & 0xFFFF0000u), acc[q][2 * i + 1]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(acc[q][i], acc[q][i], ss);
    }
  }
  // sum of squares of the row: waves, then the 4 wave sums in order
  ss = wave_sum(ss);
  if ((tid & (kWave - 1)) == 0) s_ss[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kNormThreads / kWave; ++i) tot += s_ss[i];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int q = 0; q < kNormPieces; ++q) {
    const int c = (q * kNormThreads + tid) * 8;
    if (c >= H) continue;
    const u32x4 g = *(const u32x4 *)(norm_w + c);
    u32x4 r = {0, 0, 0, 0};
    if (residual) r = *(const u32x4 *)(residual + (size_t)t * H + c);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = (__uint_as_float(r[i] << 16) + acc[q][2 * i] * inv * __uint_as_float(g[i] << 16)) * layer_scalar;
      const float hi = (__uint_as_float(r[i] & 0xFFFF0000u) +
                        acc[q][2 * i + 1] * inv * __uint_as_float(g[i] & 0xFFFF0000u)) * layer_scalar;
      o[i] = f32x2_to_bf16x2(lo, hi);
    }
    *(u32x4 *)(out + (size_t)t * H + c) = o;
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_combine_rmsnorm(const uint16_t *y_sorted, const float *topk_w,
                                   const int32_t *pair_rank, const uint16_t *norm_weight,
                                   float eps, const uint16_t *residual, float layer_scalar,
                                   int32_t T, int32_t top_k, int32_t H, uint16_t *out,
                                   void *stream) {
  using namespace moe;
  if (!norm_weight || (T > 0 && (!y_sorted || !topk_w || !pair_rank || !out))) return MOE_ERR_NULL;
  if (T < 0 || top_k <= 0 || H <= 0 || H % 8 || !(eps >= 0.0f)) return MOE_ERR_SHAPE;
  if (top_k > MOE_MAX_TOPK || H > 8 * kNormThreads * kNormPieces) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  MOE_LAUNCH(k_combine_rmsnorm, dim3(T), dim3(kNormThreads), 0, (hipStream_t)stream, y_sorted,
             topk_w, pair_rank, norm_weight, eps, residual, layer_scalar, T, top_k, H, out);
  return MOE_OK;
}

extern "C" int moe_combine(const uint16_t *y_sorted, const float *topk_w, const int32_t *pair_rank,
                           int32_t T, int32_t top_k, int32_t H, uint16_t *out, void *stream) {
  using namespace moe;
  if (T > 0 && (!y_sorted || !topk_w || !pair_rank || !out)) return MOE_ERR_NULL;
  if (T < 0 || top_k <= 0 || H <= 0 || H % 8) return MOE_ERR_SHAPE;
  if (top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  MOE_LAUNCH(k_combine, dim3(T, (H + 8 * kCombineThreads - 1) / (8 * kCombineThreads)),
             dim3(kCombineThreads), 0, (hipStream_t)stream, y_sorted, topk_w, pair_rank, T, top_k,
             H, out);
  return MOE_OK;
}
