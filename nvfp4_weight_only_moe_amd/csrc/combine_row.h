// The weighted combine of one token's routed expert outputs
// ("Gemma 4 26B-A4B (MoE) - Core AI", Architecture: sum over k of w_k h2_k)
// and its variant with the learned RMSNorm of the summed row (Architecture
// code sketch: post_feedforward_layernorm_2, the residual add, layer_scalar).
// One token row per call, shared by the two combine kernels:
//   s[c] = sum_j w[t][j] * Y[rank(t, j)][c]      (fp32 fmaf, order j = 0, 1, ...)
//   plain: out[t][c] = bf16(s[c])
//   norm:  out[t][c] = bf16((residual[t][c] + s[c] / sqrt(mean(s^2) + eps) * norm_w[c])
//                           * layer_scalar)
#pragma once
#include "common.h"

namespace moe {

// The combine + RMSNorm runs one workgroup of kNormThreads per token row:
// thread i owns columns 8(i + 256 q), q < kNormPieces.
constexpr int kNormThreads = 256;
constexpr int kNormPieces = 4;  // H <= 8 * 256 * 4 = 8192

// Ranks and weights of token t's K pairs; bit j of `valid`: rank inside [0, P).
struct TokenPairs {
  int rk[MOE_MAX_TOPK];
  float wk[MOE_MAX_TOPK];
  uint32_t valid;
};

__device__ __forceinline__ TokenPairs token_pairs(const float *__restrict__ w,
                                                  const int32_t *__restrict__ rank, int t, int K,
                                                  int P) {
  TokenPairs tp;
  tp.valid = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    tp.rk[j] = 0;
    tp.wk[j] = 0.0f;
    if (j < K) {
      const int rr = rank[(size_t)t * K + j];
      if (rr >= 0 && rr < P) {
        tp.rk[j] = rr;
        tp.wk[j] = w[(size_t)t * K + j];
        tp.valid |= 1u << j;
      }
    }
  }
  return tp;
}

// The fp32 sums of columns c .. c + 7 (c < H), accumulated in the order
// j = 0, 1, ...; the row loads of each batch of 8 pairs are all issued before
// any is used, so their latencies overlap.
constexpr int kCombineBatch = 8;
__device__ __forceinline__ void combine_sums8(const uint16_t *__restrict__ y, const TokenPairs &tp,
                                              int H, int c, float (&acc)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j0 = 0; j0 < MOE_MAX_TOPK; j0 += kCombineBatch) {
    if ((tp.valid >> j0) == 0u) break;  // no pair left
    u32x4 v[kCombineBatch];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b)
      if ((tp.valid >> (j0 + b)) & 1u) v[b] = *(const u32x4 *)(y + (size_t)tp.rk[j0 + b] * H + c);
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int j = j0 + b;
      if ((tp.valid >> j) & 1u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(tp.wk[j], __uint_as_float(v[b][i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(tp.wk[j], __uint_as_float(v[b][i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
      }
    }
  }
}

// plain combine of columns c .. c + 7 of token t (c < H)
__device__ __forceinline__ void combine_chunk(const uint16_t *__restrict__ y, const TokenPairs &tp,
                                              int H, int t, int c, uint16_t *__restrict__ out) {
  float acc[8];
  combine_sums8(y, tp, H, c, acc);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x2_to_bf16x2(acc[2 * i], acc[2 * i + 1]);
  *(u32x4 *)(out + (size_t)t * H + c) = o;
}

// combine + RMSNorm of token t's row by a workgroup of kNormThreads threads
// (tid = threadIdx.x); s_ss: LDS for kNormThreads / kWave floats.  Contains
// a barrier: every thread of the workgroup calls it.
__device__ __forceinline__ void combine_rmsnorm_row(const uint16_t *__restrict__ y,
                                                    const TokenPairs &tp,
                                                    const uint16_t *__restrict__ norm_w, float eps,
                                                    const uint16_t *residual, float layer_scalar,
                                                    int H, int t, uint16_t *out, float *s_ss) {
  const int tid = threadIdx.x;
  float acc[kNormPieces][8];
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < kNormPieces; ++q) {
    const int c = (q * kNormThreads + tid) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[q][i] = 0.0f;
    if (c < H) {
      combine_sums8(y, tp, H, c, acc[q]);
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

}  // namespace moe
