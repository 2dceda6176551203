// moe_route: the Gemma-4 MoE router on gfx950.
//
// "Gemma 4 26B-A4B (MoE) - Core AI", Architecture (router description):
// RMSNorm of the raw residual without a learned weight -> x scale x H^-0.5 ->
// linear to E logits -> softmax over all experts in fp32 -> top-k ->
// renormalise to sum 1 -> x per_expert_scale at the chosen ids.
//
// Kernel 1 (logits): the per-token factor 1/rms(x_t) * H^-0.5 is a scalar, so
//   logit[t][e] = (1/rms_t) H^-0.5 * sum_i x[t][i] * (scale[i] * W[e][i]).
// scale[i]*W[e][i] is a product of two bf16 values: exact in fp32 with at most
// 16 significant bits, so it splits exactly into hi + lo, both bf16.  Two bf16
// MFMAs (x.hi, x.lo) then give the dot product from exact products with fp32
// accumulation -- the normalised activation is never rounded to bf16.
// A workgroup owns 16 experts and 64 tokens (4 waves x 16); the hi/lo split of
// its 16 router rows is made once per K chunk in LDS and shared by the waves.
//
// Kernel 2 (select): one wave per token; softmax over all E logits in fp32,
// k rounds of a wave arg-max (ties to the lower id), renormalisation over the
// k chosen probabilities, times per_expert_scale.
#include "common.h"

namespace moe {
namespace {

constexpr int kRouteExperts = 16;   // experts per workgroup
constexpr int kRouteTokens = 64;    // tokens per workgroup (4 waves x 16)
constexpr int kRouteKC = 256;       // K chunk staged in LDS
constexpr int kRouteLdsRow = kRouteKC + 8;  // bf16 elements per LDS row (padded)

__global__ __launch_bounds__(256) void k_route_logits(const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ w,
                                                      const uint16_t *__restrict__ scale,
                                                      const float *__restrict__ bias, int T, int H,
                                                      int E, float eps,
                                                      float *__restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t s_hi[kRouteExperts * kRouteLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_lo[kRouteExperts * kRouteLdsRow];
  __shared__ float s_inv[4][16];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * kRouteExperts;
  const int t0 = blockIdx.y * kRouteTokens + wave * 16;
  const int ta = t0 + r;  // token whose A fragment this lane loads
  const bool a_ok = ta < T;
  const uint16_t *xa = x + (size_t)(a_ok ? ta : 0) * H;

  f32x4 acc_hi = {0, 0, 0, 0}, acc_lo = {0, 0, 0, 0};
  float ss = 0.0f;  // partial sum of x^2 of token ta over this lane's k

  for (int kc = 0; kc < H; kc += kRouteKC) {
    const int kcn = min(kRouteKC, H - kc);
    __syncthreads();
    // split scale[i] * W[e][i] into hi + lo (both bf16, exact)
    for (int idx = tid; idx < kRouteExperts * (kcn / 2); idx += 256) {
      const int row = idx / (kcn / 2), c2 = (idx % (kcn / 2)) * 2;
      const uint32_t wv = *(const uint32_t *)(w + (size_t)(e0 + row) * H + kc + c2);
      const uint32_t sv = *(const uint32_t *)(scale + kc + c2);
      uint32_t hi2 = 0, lo2 = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float p = bf16_to_f32((uint16_t)(wv >> (16 * h))) * bf16_to_f32((uint16_t)(sv >> (16 * h)));
        const uint16_t hb = f32_to_bf16(p);
        const uint16_t lb = f32_to_bf16(p - bf16_to_f32(hb));
        hi2 |= (uint32_t)hb << (16 * h);
        lo2 |= (uint32_t)lb << (16 * h);
      }
      *(uint32_t *)(s_hi + row * kRouteLdsRow + c2) = hi2;
      *(uint32_t *)(s_lo + row * kRouteLdsRow + c2) = lo2;
    }
    __syncthreads();
    for (int kk = 0; kk < kcn; kk += 32) {
      const int k = kk + 8 * g;
      u32x4 av = {0, 0, 0, 0};
      if (a_ok) av = *(const u32x4 *)(xa + kc + k);
      bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(av[i] << 16), hi = __uint_as_float(av[i] & 0xFFFF0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
      const bf16x8 bh = __builtin_bit_cast(bf16x8, *(const u32x4 *)(s_hi + r * kRouteLdsRow + k));
      const bf16x8 bl = __builtin_bit_cast(bf16x8, *(const u32x4 *)(s_lo + r * kRouteLdsRow + k));
      acc_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc_hi, 0, 0, 0);
      acc_lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc_lo, 0, 0, 0);
    }
  }
  // sum of squares of token r: lanes r, r+16, r+32, r+48
  ss += __shfl_xor(ss, 16, kWave);
  ss += __shfl_xor(ss, 32, kWave);
  if (g == 0) s_inv[wave][r] = 1.0f / sqrtf(ss / (float)H + eps) * (1.0f / sqrtf((float)H));
  __syncthreads();
  // C layout: lane holds rows (tokens) 4g+j, column (expert) r
  const int e = e0 + r;
  const float b = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 4 * g + j;
    if (t < T) logits[(size_t)t * E + e] = (acc_hi[j] + acc_lo[j]) * s_inv[wave][4 * g + j] + b;
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
  m = wave_max(m);
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) z += (lane + i * kWave < E) ? expf(v[i] - m) : 0.0f;
  z = wave_sum(z);
  const float inv_z = 1.0f / z;

  uint32_t taken = 0;  // bit i: my element lane + 64 i is already chosen
  int my_id = -1;      // lane j (< K) keeps the j-th selection
  float my_p = 0.0f;
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
    const float p = expf(bv - m) * inv_z;
    psum += p;
    if (lane == s) {
      my_id = bi;
      my_p = p;
    }
  }
  if (lane < K) {
    const float wr = my_p / psum;
    topk_idx[(size_t)t * K + lane] = my_id;
    topk_w[(size_t)t * K + lane] = wr * bf16_to_f32(pes[my_id]);
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
  if (E > MOE_MAX_EXPERTS || E % kRouteExperts || top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  dim3 g1(E / kRouteExperts, (T + kRouteTokens - 1) / kRouteTokens);
  MOE_LAUNCH(k_route_logits, g1, dim3(256), 0, s, x, w_router, router_scale, logit_bias, T,
                     H, E, eps, logits);
  MOE_LAUNCH(k_route_select, dim3((T + 3) / 4), dim3(256), 0, s, logits, per_expert_scale,
                     T, E, top_k, topk_idx, topk_w, topk_w_raw);
  return MOE_OK;
}
