// The weighted combine of one token's routed expert outputs
// ("Gemma 4 26B-A4B (MoE) - Core AI", Architecture: sum over k of w_k h2_k)
// and its variant with the learned norms of the layer step that follows
// (Architecture code sketch: post_feedforward_layernorm_2 of the sum, then
// the residual plus post_feedforward_layernorm of h1 + h2, times
// layer_scalar).  One token row per call, shared by the two combine kernels:
//   s[c]  = sum_j w[t][j] * Y[rank(t, j)][c]   (fp32 fmaf, order j = 0, 1, ...)
//   plain: out[t][c] = bf16(s[c])
//   norm:  h2 = s / sqrt(mean(s^2) + eps) * w2            (fp32)
//          branch only: out = bf16(h2)
//          layer step:  u = h1 + h2;
//                       out = bf16((residual + u / sqrt(mean(u^2) + eps) * w) * layer_scalar)
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
// any is used, so their latencies overlap.  The expert outputs are read once:
// non-temporal loads keep them from displacing other data in the caches
// (16384 tokens: combine 186 -> 145 us).
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
      if ((tp.valid >> (j0 + b)) & 1u)
        v[b] = __builtin_nontemporal_load((const u32x4 *)(y + (size_t)tp.rk[j0 + b] * H + c));
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

// Sum of v over a workgroup of kNormThreads threads, the same in every
// thread: wave sums, then the wave sums in wave order.  s_part: LDS for
// kNormThreads / kWave floats, not in use by another reduction.
__device__ __forceinline__ float block_sum(float v, float *s_part) {
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) s_part[threadIdx.x / kWave] = v;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kNormThreads / kWave; ++i) tot += s_part[i];
  return tot;
}

__device__ __forceinline__ void unpack8(const u32x4 &v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

// The combine and the layer step's norms for token t's row by a workgroup of
// kNormThreads threads (tid = threadIdx.x): norm2_w is the weight of the norm
// of the summed row (h2); with norm_w the layer step follows (h1 may be
// NULL: zero; residual is then required), else the row is h2.  s_ss: LDS for
// 2 * kNormThreads / kWave floats.  Contains barriers: every thread of the
// workgroup calls it.  h1, residual and out may be the same buffer: each
// element is read before it is written, by one thread.
__device__ __forceinline__ void combine_layer_row(const uint16_t *__restrict__ y,
                                                  const TokenPairs &tp,
                                                  const uint16_t *__restrict__ norm2_w,
                                                  const uint16_t *h1,
                                                  const uint16_t *__restrict__ norm_w,
                                                  const uint16_t *residual, float eps,
                                                  float layer_scalar, int H, int t, uint16_t *out,
                                                  float *s_ss) {
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
  // h2 = rmsnorm(s, norm2_w)
  const float inv2 = 1.0f / sqrtf(block_sum(ss, s_ss) / (float)H + eps);
  float ss2 = 0.0f;
#pragma unroll
  for (int q = 0; q < kNormPieces; ++q) {
    const int c = (q * kNormThreads + tid) * 8;
    if (c >= H) continue;
    float g[8], a[8];
    unpack8(*(const u32x4 *)(norm2_w + c), g);
    if (norm_w && h1) unpack8(*(const u32x4 *)(h1 + (size_t)t * H + c), a);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[q][i] = acc[q][i] * inv2 * g[i];
      if (norm_w && h1) acc[q][i] += a[i];  // u = h1 + h2
      ss2 = fmaf(acc[q][i], acc[q][i], ss2);
    }
  }
  float inv = 1.0f;
  if (norm_w) inv = 1.0f / sqrtf(block_sum(ss2, s_ss + kNormThreads / kWave) / (float)H + eps);
#pragma unroll
  for (int q = 0; q < kNormPieces; ++q) {
    const int c = (q * kNormThreads + tid) * 8;
    if (c >= H) continue;
    u32x4 o;
    if (!norm_w) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = f32x2_to_bf16x2(acc[q][2 * i], acc[q][2 * i + 1]);
    } else {
      float g[8], r[8];
      unpack8(*(const u32x4 *)(norm_w + c), g);
      unpack8(*(const u32x4 *)(residual + (size_t)t * H + c), r);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = f32x2_to_bf16x2((r[2 * i] + acc[q][2 * i] * inv * g[2 * i]) * layer_scalar,
                               (r[2 * i + 1] + acc[q][2 * i + 1] * inv * g[2 * i + 1]) * layer_scalar);
    }
    *(u32x4 *)(out + (size_t)t * H + c) = o;
  }
}

}  // namespace moe
