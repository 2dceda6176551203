// moe_route: the Gemma-4 MoE router on gfx950.
//
// "Gemma 4 26B-A4B (MoE) - Core AI", Architecture (router description):
// RMSNorm of the raw residual without a learned weight -> x scale x H^-0.5 ->
// linear to E logits -> softmax over all experts in fp32 -> top-k ->
// renormalise to sum 1 -> x per_expert_scale at the chosen ids.
//
// Kernel 1 (logits): the per-token factor 1/rms(x_t) * H^-0.5 is a scalar, so
//   logit[t][e] = (1/rms_t) H^-0.5 * sum_i x[t][i] * scale[i] * W[e][i].
// A product of two bf16 values is exact in fp32 (at most 16 significant bits)
// and splits exactly into hi + lo, both bf16; with it each term x*scale*W is
// formed exactly by two bf16 MFMAs and summed in fp32 -- the normalised
// activation is never rounded to bf16.  Two tilings:
//  * few tokens (T <= 64): the split is taken on the weight side,
//    scale*W = hi + lo, and x is the MFMA operand as it is; a workgroup owns
//    16 experts and all tokens, its 8 waves split K and meet in LDS.
//  * many tokens: the split is taken on the activation side,
//    x*scale = hi + lo, W is the operand as it is; a workgroup owns 64 tokens
//    (4 waves x 16) and NF*16 experts per wave, full K.
//
// Kernel 2 (select): one wave per token; softmax over all E logits in fp32,
// k rounds of a wave arg-max (ties to the lower id), renormalisation over the
// k chosen probabilities, times per_expert_scale.
#include "common.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// 8 bf16 a (as 4 dwords) times 8 bf16 b, each product split exactly into
// hi + lo bf16 (hardware round-to-nearest-even conversion of pairs).
__device__ __forceinline__ void split_products(const u32x4 &a, const u32x4 &b, bf16x8 &hi,
                                               bf16x8 &lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 p = {__uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16),
                     __uint_as_float(a[i] & 0xFFFF0000u) * __uint_as_float(b[i] & 0xFFFF0000u)};
    const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
    const f32x2 r = {p[0] - __uint_as_float(hb << 16), p[1] - __uint_as_float(hb & 0xFFFF0000u)};
    h[i] = hb;
    l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ float sumsq8(const u32x4 &v) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- few tokens: 16 experts per workgroup, 8 waves split K, MT x 16 tokens
constexpr int kNarrowWaves = 8;

template <int MT>
__global__ __launch_bounds__(kNarrowWaves * 64) void k_route_logits_narrow(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const uint16_t *__restrict__ scale, const float *__restrict__ bias, int T, int H, int E,
    float eps, float *__restrict__ logits) {
  __shared__ f32x4 s_acc[kNarrowWaves][MT][64];
  __shared__ float s_ss[kNarrowWaves][MT * 16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 16;
  const uint16_t *wrow = w + (size_t)(e0 + r) * H;
  f32x4 acc[MT];
  float ss[MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    acc[q] = f32x4{0, 0, 0, 0};
    ss[q] = 0.0f;
  }
  // k-steps of 32 are dealt to the waves round-robin; each lane issues the
  // loads of kBatch steps before using any of them
  constexpr int kBatch = 4;
  const int nsteps = H / 32;
  for (int ks0 = wave; ks0 < nsteps; ks0 += kNarrowWaves * kBatch) {
    u32x4 wv[kBatch], sv[kBatch], xv[kBatch][MT];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int ks = ks0 + b * kNarrowWaves;
      const int k = ks * 32 + 8 * g;
      wv[b] = sv[b] = u32x4{0, 0, 0, 0};
      if (ks < nsteps) {
        wv[b] = *(const u32x4 *)(wrow + k);
        sv[b] = *(const u32x4 *)(scale + k);
      }
#pragma unroll
      for (int q = 0; q < MT; ++q) {
        const int t = q * 16 + r;
        xv[b][q] = u32x4{0, 0, 0, 0};
        if (ks < nsteps && t < T) xv[b][q] = *(const u32x4 *)(x + (size_t)t * H + k);
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (ks0 + b * kNarrowWaves < nsteps) {  // uniform across the wave
        bf16x8 bh, bl;
        split_products(wv[b], sv[b], bh, bl);
#pragma unroll
        for (int q = 0; q < MT; ++q) {
          ss[q] += sumsq8(xv[b][q]);
          const bf16x8 a = __builtin_bit_cast(bf16x8, xv[b][q]);
          acc[q] = mfma_bf16(a, bh, acc[q]);
          acc[q] = mfma_bf16(a, bl, acc[q]);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    s_acc[wave][q][lane] = acc[q];
    float v = ss[q];  // x^2 of token q*16 + r over this lane's k
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    if (g == 0) s_ss[wave][q * 16 + r] = v;
  }
  __syncthreads();
  if (wave != 0) return;
  const float hs = 1.0f / sqrtf((float)H);
  const float b = bias ? bias[e0 + r] : 0.0f;
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    f32x4 tot = {0, 0, 0, 0};
    for (int v = 0; v < kNarrowWaves; ++v) tot += s_acc[v][q][lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = q * 16 + 4 * g + j, t = m;
      if (t < T) {
        float sq = 0.0f;
        for (int v = 0; v < kNarrowWaves; ++v) sq += s_ss[v][m];
        const float inv = 1.0f / sqrtf(sq / (float)H + eps) * hs;
        logits[(size_t)t * E + e0 + r] = tot[j] * inv + b;
      }
    }
  }
}

// ---- many tokens: 64 tokens per workgroup, NF*16 experts per wave
template <int NF>
__global__ __launch_bounds__(256) void k_route_logits_wide(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const uint16_t *__restrict__ scale, const float *__restrict__ bias, int T, int H, int E,
    float eps, float *__restrict__ logits) {
  __shared__ float s_inv[4][16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * NF * 16;
  const int t0 = blockIdx.y * 64 + wave * 16;
  const int ta = t0 + r;
  const bool a_ok = ta < T;
  const uint16_t *xa = x + (size_t)(a_ok ? ta : 0) * H;
  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0, 0, 0, 0};
  float ss = 0.0f;
  for (int kk = 0; kk < H; kk += 32) {
    const int k = kk + 8 * g;
    u32x4 xv = {0, 0, 0, 0};
    if (a_ok) xv = *(const u32x4 *)(xa + k);
    const u32x4 sv = *(const u32x4 *)(scale + k);
    ss += sumsq8(xv);
    bf16x8 ah, al;
    split_products(xv, sv, ah, al);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, *(const u32x4 *)(w + (size_t)(e0 + f * 16 + r) * H + k));
      acc[f] = mfma_bf16(ah, b, acc[f]);
      acc[f] = mfma_bf16(al, b, acc[f]);
    }
  }
  ss += __shfl_xor(ss, 16, kWave);
  ss += __shfl_xor(ss, 32, kWave);
  if (g == 0) s_inv[wave][r] = 1.0f / sqrtf(ss / (float)H + eps) * (1.0f / sqrtf((float)H));
  __syncthreads();
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int e = e0 + f * 16 + r;
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + 4 * g + j;
      if (t < T) logits[(size_t)t * E + e] = acc[f][j] * s_inv[wave][4 * g + j] + b;
    }
  }
}

__global__ __launch_bounds__(256) void k_route_select(const float *__restrict__ logits,
                                                      const uint16_t *__restrict__ pes, int T,
                                                      int E, int K, int32_t *__restrict__ topk_idx,
                                                      float *__restrict__ topk_w,
                                                      float *__restrict__ topk_w_raw) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *lg = logits + (size_t)t * E;
  constexpr int kPer = MOE_MAX_EXPERTS / kWave;  // 4
  float v[kPer];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + i * kWave;
    v[i] = e < E ? lg[e] : -__builtin_huge_valf();
    m = fmaxf(m, v[i]);
  }
  // per_expert_scale of this lane's experts, loaded up front (no dependent
  // load after the selection)
  float pv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + i * kWave;
    pv[i] = e < E ? bf16_to_f32(pes[e]) : 0.0f;
  }
  m = wave_max(m);
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) z += (lane + i * kWave < E) ? expf(v[i] - m) : 0.0f;
  z = wave_sum(z);
  const float inv_z = 1.0f / z;

  uint32_t taken = 0;  // bit i: my element lane + 64 i is already chosen
  int my_id = -1;      // lane j (< K) keeps the j-th selection
  float my_p = 0.0f, my_pes = 0.0f;
  float psum = 0.0f;
  for (int s = 0; s < K; ++s) {
    // lane-local best (largest logit, lowest id among equals)
    float bv = -__builtin_huge_valf();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + i * kWave;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    // per_expert_scale of the winner, from the lane that holds it
    float pw = pv[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i)
      if (bi / kWave == i) pw = pv[i];
    pw = __shfl(pw, bi & (kWave - 1), kWave);
    const float p = expf(bv - m) * inv_z;
    psum += p;
    if (lane == s) {
      my_id = bi;
      my_p = p;
      my_pes = pw;
    }
  }
  if (lane < K) {
    const float wr = my_p / psum;
    topk_idx[(size_t)t * K + lane] = my_id;
    topk_w[(size_t)t * K + lane] = wr * my_pes;
    if (topk_w_raw) topk_w_raw[(size_t)t * K + lane] = wr;
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_route(const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
                         const uint16_t *per_expert_scale, const float *logit_bias, int32_t T,
                         int32_t H, int32_t E, int32_t top_k, float eps, int32_t *topk_idx,
                         float *topk_w, float *topk_w_raw, float *logits, void *stream) {
  using namespace moe;
  if (!w_router || !router_scale || !per_expert_scale) return MOE_ERR_NULL;
  if (T > 0 && (!x || !topk_idx || !topk_w || !logits)) return MOE_ERR_NULL;
  if (T < 0 || H <= 0 || H % 32 || E <= 0 || top_k <= 0 || top_k > E) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS || E % 16 || top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (T <= 64) {
    const dim3 grid(E / 16), block(kNarrowWaves * 64);
    const int mt = (T + 15) / 16;
    if (mt == 1)
      MOE_LAUNCH(k_route_logits_narrow<1>, grid, block, 0, s, x, w_router, router_scale, logit_bias, T, H, E, eps, logits);
    else if (mt == 2)
      MOE_LAUNCH(k_route_logits_narrow<2>, grid, block, 0, s, x, w_router, router_scale, logit_bias, T, H, E, eps, logits);
    else
      MOE_LAUNCH(k_route_logits_narrow<4>, grid, block, 0, s, x, w_router, router_scale, logit_bias, T, H, E, eps, logits);
  } else {
    // experts per workgroup: all of them (NF = E/16 up to 8) unless that
    // leaves too few workgroups
    const int tg = (T + 63) / 64;
    const bool wide8 = (E % 128 == 0) && tg >= 128;
    if (wide8)
      MOE_LAUNCH(k_route_logits_wide<8>, dim3(E / 128, tg), dim3(256), 0, s, x, w_router, router_scale, logit_bias, T, H, E, eps, logits);
    else
      MOE_LAUNCH(k_route_logits_wide<1>, dim3(E / 16, tg), dim3(256), 0, s, x, w_router, router_scale, logit_bias, T, H, E, eps, logits);
  }
  MOE_LAUNCH(k_route_select, dim3((T + 3) / 4), dim3(256), 0, s, logits, per_expert_scale,
                     T, E, top_k, topk_idx, topk_w, topk_w_raw);
  return MOE_OK;
}
