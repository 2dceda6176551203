// moe_combine: weighted sum of a token's routed expert outputs
// ("Gemma 4 26B-A4B (MoE) - Core AI", Architecture: sum over k of w_k h2_k).
// out[t] = sum_j w[t][j] * Y[rank(t, j)], fixed order j = 0, 1, ..., fp32
// accumulation, one bf16 rounding.  Workgroup (t, c) covers token t's columns
// 1024c .. 1024c + 1023; each thread owns 8 consecutive outputs (16-byte
// loads and stores), so even a decode batch spreads over many workgroups.
#include "combine_row.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 128;

__global__ __launch_bounds__(kCombineThreads) void k_combine(const uint16_t *__restrict__ y,
                                                 const float *__restrict__ w,
                                                 const int32_t *__restrict__ rank, int T, int K,
                                                 int H, uint16_t *__restrict__ out) {
  const int t = blockIdx.x;
  // ranks and weights first, then every row load issued before any is used
  const TokenPairs tp = token_pairs(w, rank, t, K, T * K);
  const int c = (blockIdx.y * kCombineThreads + threadIdx.x) * 8;
  if (c < H) combine_chunk(y, tp, H, t, c, out);
}

// The combine followed by the layer step's learned norms: one workgroup per
// token (a norm needs the whole row), the row kept in registers between the
// sums of squares and the output.
__global__ __launch_bounds__(kNormThreads) void k_combine_rmsnorm(
    const uint16_t *__restrict__ y, const float *__restrict__ w, const int32_t *__restrict__ rank,
    const uint16_t *__restrict__ norm2_w, const uint16_t *h1, const uint16_t *__restrict__ norm_w,
    const uint16_t *residual, float eps, float layer_scalar, int T, int K, int H, uint16_t *out) {
  __shared__ float s_ss[2 * kNormThreads / kWave];
  const int t = blockIdx.x;
  const TokenPairs tp = token_pairs(w, rank, t, K, T * K);
  combine_layer_row(y, tp, norm2_w, h1, norm_w, residual, eps, layer_scalar, H, t, out, s_ss);
}

}  // namespace
}  // namespace moe

extern "C" int moe_combine_rmsnorm(const uint16_t *y_sorted, const float *topk_w,
                                   const int32_t *pair_rank, const uint16_t *post_norm2_weight,
                                   const uint16_t *h1, const uint16_t *post_norm_weight,
                                   const uint16_t *residual, float eps, float layer_scalar,
                                   int32_t T, int32_t top_k, int32_t H, uint16_t *out,
                                   void *stream) {
  using namespace moe;
  if (!post_norm2_weight || (post_norm_weight && T > 0 && !residual)) return MOE_ERR_NULL;
  if (T > 0 && (!y_sorted || !topk_w || !pair_rank || !out)) return MOE_ERR_NULL;
  if (!post_norm_weight && (h1 || residual)) return MOE_ERR_SHAPE;
  if (T < 0 || top_k <= 0 || H <= 0 || H % 8 || !(eps >= 0.0f)) return MOE_ERR_SHAPE;
  if (top_k > MOE_MAX_TOPK || H > 8 * kNormThreads * kNormPieces) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  MOE_LAUNCH(k_combine_rmsnorm, dim3(T), dim3(kNormThreads), 0, (hipStream_t)stream, y_sorted,
             topk_w, pair_rank, post_norm2_weight, h1, post_norm_weight, residual, eps,
             layer_scalar, T, top_k, H, out);
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
