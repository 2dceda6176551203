// moe_route: the Gemma-4 MoE router on gfx950.
//
// "Gemma 4 26B-A4B (MoE) - Core AI", Architecture (router description):
// RMSNorm of the raw residual without a learned weight -> x scale x H^-0.5 ->
// linear to E logits -> softmax over all experts in fp32 -> top-k ->
// renormalise to sum 1 -> x per_expert_scale at the chosen ids.
//
// Kernel 1 (logits): the per-token factor 1/rms(x_t) * H^-0.5 is a scalar, so
//   logit[t][e] = (1/rms_t) H^-0.5 * sum_i x[t][i] * scale[i] * W[e][i],
// every term formed exactly and summed in fp32 -- the normalised activation
// is never rounded to bf16.  Two tilings:
//  * few tokens (T <= 64): plain fp32 FMAs, no LDS.  x*scale*W is a product
//    of three bf16 values (at most 24 significant bits), exact in fp32.  A
//    workgroup owns one expert and 16 tokens, each wave 4 of them, the whole
//    row of scale*W kept in registers.
//  * many tokens: bf16 MFMAs.  The product of two bf16 values is exact in
//    fp32 and splits exactly into hi + lo, both bf16: x*scale = hi + lo is
//    staged in LDS, W is the operand as it is, two MFMAs per term.  A
//    workgroup owns 64 tokens (4 waves x 16) and EXP experts, full K.  With
//    no logits buffer the workgroup holds every expert, keeps the logits in
//    LDS and selects there (kernel 2 folded in).
//
// Kernel 2 (select): one wave per token; softmax over all E logits in fp32,
// k rounds of a wave arg-max (ties to the lower id), renormalisation over the
// k chosen probabilities, times per_expert_scale.
#include "common.h"
#include "select.h"

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

// ---- few tokens (T <= 64): plain fp32 FMAs.  x*scale*W is a product of
// three bf16 values, at most 24 significant bits: exact in fp32, so fma()
// adds exact products with one rounding each, as the MFMA path does.  A
// workgroup owns one expert; each wave keeps scale*W of the whole row in
// registers (exact) and takes up to 16 tokens; every load is a coalesced
// 16-byte-per-lane read along a row.
constexpr int kFewMaxV = 8;  // 16-byte vectors per lane: H <= 64 * 8 * kFewMaxV

// With pa.x16 (the fused decode layer), ceil(T/4) more workgroups in the row
// y = 0 (blockIdx.x >= E) write the expert input's f16 rows (one wave per
// token) and clear the per-row maximum of A.
template <int NV>  // 16-byte vectors per lane: lane holds k = (v*64 + lane)*8 .. +7
__global__ __launch_bounds__(256) void k_route_logits_few(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const uint16_t *__restrict__ scale, const float *__restrict__ bias, int T, int H, int E,
    float eps, float *__restrict__ logits, int32_t *__restrict__ arrive, PrepArgs pa) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (e >= E) {  // the expert-input prep (uniform per workgroup)
    if (blockIdx.y != 0) return;
    const int wg = e - E;
    for (int i = wg * 256 + threadIdx.x; i < pa.P; i += 256 * ((T + 3) / 4)) pa.a_max[i] = 0u;
    const int t = wg * 4 + wave;
    if (t < T) {
      if (pa.norm_w)
        prep_row<true>(pa.x, pa.norm_w, pa.norm_eps, pa.H, t, pa.x16, pa.x_exp);
      else
        prep_row<false>(pa.x, nullptr, 0.0f, pa.H, t, pa.x16, pa.x_exp);
    }
    return;
  }
  // the arrival counter of the selection kernel that follows (when given)
  if (arrive && e == 0 && blockIdx.y == 0 && threadIdx.x == 0) *arrive = 0;
  // workgroup (e, y) takes tokens 16y .. 16y+15, 4 per wave
  constexpr int kTPW = 4;
  const int t0 = blockIdx.y * 16 + wave * kTPW;
  // every load first (the W row, the scale and the wave's token rows do not
  // depend on each other, so their latencies overlap); lanes past H read row
  // start 0 and are masked below
  int koff[NV];
  u32x4 wv[NV], sv[NV], xv[kTPW][NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int k = (v * 64 + lane) * 8;
    koff[v] = k < H ? k : 0;
    wv[v] = *(const u32x4 *)(w + (size_t)e * H + koff[v]);
    sv[v] = *(const u32x4 *)(scale + koff[v]);
  }
#pragma unroll
  for (int q = 0; q < kTPW; ++q) {
    const int t = min(t0 + q, T - 1);
#pragma unroll
    for (int v = 0; v < NV; ++v) xv[q][v] = *(const u32x4 *)(x + (size_t)t * H + koff[v]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // scale*W of this lane's K elements (exact in fp32); lanes past H hold 0
  float sw[NV * 8];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const bool ok = (v * 64 + lane) * 8 < H;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = __uint_as_float(wv[v][i] << 16) * __uint_as_float(sv[v][i] << 16);
      const float p1 =
          __uint_as_float(wv[v][i] & 0xFFFF0000u) * __uint_as_float(sv[v][i] & 0xFFFF0000u);
      sw[v * 8 + 2 * i] = ok ? p0 : 0.0f;
      sw[v * 8 + 2 * i + 1] = ok ? p1 : 0.0f;
    }
  }
  const float hs = 1.0f / sqrtf((float)H);
  const float b = bias ? bias[e] : 0.0f;
  float dot[kTPW], ss[kTPW];
#pragma unroll
  for (int q = 0; q < kTPW; ++q) {
    dot[q] = ss[q] = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const bool ok = (v * 64 + lane) * 8 < H;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = ok ? __uint_as_float(xv[q][v][i] << 16) : 0.0f;
        const float hi = ok ? __uint_as_float(xv[q][v][i] & 0xFFFF0000u) : 0.0f;
        dot[q] = fmaf(lo, sw[v * 8 + 2 * i], dot[q]);
        dot[q] = fmaf(hi, sw[v * 8 + 2 * i + 1], dot[q]);
        ss[q] = fmaf(lo, lo, ss[q]);
        ss[q] = fmaf(hi, hi, ss[q]);
      }
    }
  }
  // wave sums (DPP rows, then the four rows; uniform results); lane q writes token q
  float d = 0.0f, q2 = 0.0f;
#pragma unroll
  for (int q = 0; q < kTPW; ++q) {
    const float dq = wave_sum_u(dot[q]), sq = wave_sum_u(ss[q]);
    if (lane == q) {
      d = dq;
      q2 = sq;
    }
  }
  const int t = t0 + lane;
  if (lane < kTPW && t < T)
    logits[(size_t)t * E + e] = d * (1.0f / sqrtf(q2 / (float)H + eps) * hs) + b;
}

// ---- many tokens: 64 tokens x EXP experts per workgroup (16 x EXP per wave;
// EXP = 16 or 32, the smaller tile doubling the workgroups of mid-sized
// batches at the cost of staging each token chunk twice as often).  K in
// chunks of 128 staged in LDS by coalesced row loads (16 threads per row); the
// next chunk is loaded into registers while the current one is multiplied.
// The split is taken on the activation side when staging: x*scale = hi + lo
// (both bf16, exact).
constexpr int kWideKC = 128;
constexpr int kWideTok = 64;
constexpr int kWideLd = kWideKC + 8;  // bf16 per LDS row (padding spreads banks)
// below this many tokens the 16-expert tile (T = 128: step 130 -> 127 us,
// T = 512: 232 -> 228 us; T = 2048 unchanged, T = 16384 slower)
constexpr int kWideExp16Below = 2048;

// SELECT (moe_route without a logits buffer): one workgroup holds every
// expert (EXP >= E) of its 64 tokens, writes their logits into LDS (over the
// weight staging area, free after the K loop) instead of memory, and its
// waves then select for the tokens from there.
// SPLIT (K-split, moe_route_bucket): workgroup z of gridDim.z takes K chunks
// [z n / Z, (z + 1) n / Z) and writes its raw dot products into part[z][t][e]
// and (expert block 0) the token's sum of squares over them into pss[z][t];
// k_route_select_split finishes the logits.
template <int EXP, bool SELECT, bool SPLIT = false>
__global__ __launch_bounds__(256) void k_route_logits_wide(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const uint16_t *__restrict__ scale, const float *__restrict__ bias, int T, int H, int E,
    float eps, float *__restrict__ logits, const uint16_t *__restrict__ pes, int K,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ topk_w_raw,
    float *__restrict__ part, float *__restrict__ pss) {
  __shared__ __attribute__((aligned(16))) uint16_t s_xh[kWideTok * kWideLd];
  __shared__ __attribute__((aligned(16))) uint16_t s_xl[kWideTok * kWideLd];
  constexpr int NF = EXP / 16;  // 16-expert MFMA column tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t s_w[EXP * kWideLd];
  __shared__ float s_ss[kWideTok];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * EXP;
  const int t0 = blockIdx.y * kWideTok;
  // staging map: 16 threads per row, rows srow + 16h
  const int srow = tid >> 4, scol = (tid & 15) * 8;
  const uint16_t *xrow[4];
  bool xok[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int t = t0 + srow + 16 * h;
    xok[h] = t < T;
    xrow[h] = x + (size_t)(xok[h] ? t : 0) * H;
  }
  const uint16_t *wrow[NF];
  bool wok[NF];
#pragma unroll
  for (int h = 0; h < NF; ++h) {
    const int ee = e0 + srow + 16 * h;
    wok[h] = ee < E;
    wrow[h] = w + (size_t)(wok[h] ? ee : 0) * H;
  }
  u32x4 xv[4], wv[NF], sv;
  auto load = [&](int kc) {
    const bool kok = kc + scol < H;  // chunks past the end (H % 128 = 64, or the last prefetch) read zeros
    const u32x4 s0 = *(const u32x4 *)(scale + (kok ? kc + scol : 0));
    sv = kok ? s0 : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 v = *(const u32x4 *)(xrow[h] + (kok ? kc + scol : 0));
      xv[h] = (xok[h] && kok) ? v : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int h = 0; h < NF; ++h) {
      const u32x4 v = *(const u32x4 *)(wrow[h] + (kok ? kc + scol : 0));
      wv[h] = (wok[h] && kok) ? v : u32x4{0, 0, 0, 0};
    }
  };
  float ss[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto store = [&]() {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      ss[h] += sumsq8(xv[h]);
      bf16x8 hi, lo;
      split_products(xv[h], sv, hi, lo);
      *(bf16x8 *)(s_xh + (srow + 16 * h) * kWideLd + scol) = hi;
      *(bf16x8 *)(s_xl + (srow + 16 * h) * kWideLd + scol) = lo;
    }
#pragma unroll
    for (int h = 0; h < NF; ++h) *(u32x4 *)(s_w + (srow + 16 * h) * kWideLd + scol) = wv[h];
  };
  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0, 0, 0, 0};
  const int nchunks = (H + kWideKC - 1) / kWideKC;
  const int cb = SPLIT ? (int)(blockIdx.z * nchunks / gridDim.z) : 0;
  const int ce = SPLIT ? (int)((blockIdx.z + 1) * nchunks / gridDim.z) : nchunks;
  // the chunk past ce (the last prefetch) reads zeros, or the next slice's
  // first chunk, which is never stored
  load(cb * kWideKC);
  for (int kc = cb * kWideKC; kc < ce * kWideKC; kc += kWideKC) {
    store();
    __syncthreads();
    load(kc + kWideKC);  // next chunk in flight during the MFMAs
#pragma unroll
    for (int ks = 0; ks < kWideKC; ks += 32) {
      const int k = ks + 8 * g;
      const bf16x8 ah = *(const bf16x8 *)(s_xh + (wave * 16 + r) * kWideLd + k);
      const bf16x8 al = *(const bf16x8 *)(s_xl + (wave * 16 + r) * kWideLd + k);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const bf16x8 b = *(const bf16x8 *)(s_w + (f * 16 + r) * kWideLd + k);
        acc[f] = mfma_bf16(ah, b, acc[f]);
        acc[f] = mfma_bf16(al, b, acc[f]);
      }
    }
    __syncthreads();
  }
  // sum of squares per token: 16 threads per row
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float v = ss[h];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, kWave);
    if ((tid & 15) == 0) s_ss[srow + 16 * h] = v;
  }
  __syncthreads();
  if (SPLIT) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int e = e0 + f * 16 + r;
      if (e >= E) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + wave * 16 + 4 * g + j;
        if (t < T) part[((size_t)blockIdx.z * T + t) * E + e] = acc[f][j];
      }
    }
    if (blockIdx.x == 0 && tid < kWideTok && t0 + tid < T) pss[(size_t)blockIdx.z * T + t0 + tid] = s_ss[tid];
    return;
  }
  const float hs = 1.0f / sqrtf((float)H);
  static_assert(!SELECT || EXP * kWideLd * 2 >= kWideTok * EXP * 4, "LDS logits fit the W area");
  float *s_logit = reinterpret_cast<float *>(s_w);  // SELECT: [kWideTok][E]
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int e = e0 + f * 16 + r;
    if (e >= E) continue;
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = wave * 16 + 4 * g + j, t = t0 + m;
      const float v = acc[f][j] * (1.0f / sqrtf(s_ss[m] / (float)H + eps) * hs) + b;
      if (SELECT) s_logit[m * E + e] = v;
      else if (t < T) logits[(size_t)t * E + e] = v;
    }
  }
  if (SELECT) {
    __syncthreads();
    for (int m = wave; m < kWideTok && t0 + m < T; m += 4)
      select_token_n<(EXP + kWave - 1) / kWave, true>(s_logit + m * E, pes, t0 + m, E, K,
                                                      topk_idx, topk_w, topk_w_raw);
  }
}

// The K-split router's end: one wave per token adds the ks partial dot
// products and sums of squares in slice order, scales them as the unsplit
// kernel does, writes the logits (when asked) and selects from them.
constexpr int kRouteMaxKs = 8;  // route_split_cfg's most slices
template <int NPER>
__global__ __launch_bounds__(256) void k_route_select_split(
    const float *__restrict__ part, const float *__restrict__ pss, int ks,
    const float *__restrict__ bias, int T, int H, int E, float eps, float *__restrict__ logits,
    const uint16_t *__restrict__ pes, int K, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, float *__restrict__ topk_w_raw) {
  __shared__ float s_row[4][NPER * kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t < T) {
    // every partial load issued before the first add (ks <= kRouteMaxKs)
    float pz[kRouteMaxKs], vz[NPER][kRouteMaxKs];
#pragma unroll
    for (int z = 0; z < kRouteMaxKs; ++z) {
      pz[z] = z < ks ? pss[(size_t)z * T + t] : 0.0f;
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const int e = lane + i * kWave;
        vz[i][z] = (z < ks && e < E) ? part[((size_t)z * T + t) * E + e] : 0.0f;
      }
    }
    float ss = 0.0f;
#pragma unroll
    for (int z = 0; z < kRouteMaxKs; ++z)
      if (z < ks) ss += pz[z];
    const float f = 1.0f / sqrtf(ss / (float)H + eps) * (1.0f / sqrtf((float)H));
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = lane + i * kWave;
      if (e >= E) break;
      float a = 0.0f;
#pragma unroll
      for (int z = 0; z < kRouteMaxKs; ++z)
        if (z < ks) a += vz[i][z];
      const float v = a * f + (bias ? bias[e] : 0.0f);
      if (logits) logits[(size_t)t * E + e] = v;
      s_row[wave][e] = v;
    }
  }
  __syncthreads();
  if (t < T) select_token_n<NPER, true>(s_row[wave], pes, t, E, K, topk_idx, topk_w, topk_w_raw);
}

__global__ __launch_bounds__(256) void k_route_select(const float *__restrict__ logits,
                                                      const uint16_t *__restrict__ pes, int T,
                                                      int E, int K, int32_t *__restrict__ topk_idx,
                                                      float *__restrict__ topk_w,
                                                      float *__restrict__ topk_w_raw) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  select_token(logits, pes, t, E, K, topk_idx, topk_w, topk_w_raw);
}

}  // namespace
}  // namespace moe

namespace moe {
// moe_route_bucket: up to kFusedMaxT tokens the selection runs over many
// workgroups and the last one to finish buckets, in one launch.
constexpr int kFusedMaxT = 64;
int launch_select_bucket(const float *logits, const uint16_t *pes, int T, int E, int top_k,
                         int32_t *topk_idx, float *topk_w, float *topk_w_raw,
                         int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_rank,
                         void *workspace, const PrepArgs &pa, hipStream_t s);
}

extern "C" int moe_route(const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
                         const uint16_t *per_expert_scale, const float *logit_bias, int32_t T,
                         int32_t H, int32_t E, int32_t top_k, float eps, int32_t *topk_idx,
                         float *topk_w, float *topk_w_raw, float *logits, void *stream) {
  using namespace moe;
  if (!w_router || !router_scale || !per_expert_scale) return MOE_ERR_NULL;
  if (T > 0 && (!x || !topk_idx || !topk_w)) return MOE_ERR_NULL;
  if (T < 0 || H <= 0 || H % 64 || E <= 0 || top_k <= 0 || top_k > E) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS || E % 16 || top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (!logits) {  // logits kept in LDS: one workgroup per 64 tokens holds every expert
    const dim3 grid(1, (T + kWideTok - 1) / kWideTok);
#define MOE_ALL(EXP)                                                                            \
  MOE_LAUNCH((k_route_logits_wide<EXP, true>), grid, dim3(256), 0, s, x, w_router, router_scale, \
             logit_bias, T, H, E, eps, (float *)nullptr, per_expert_scale, top_k, topk_idx,       \
             topk_w, topk_w_raw, (float *)nullptr, (float *)nullptr)
    if (E <= 64) MOE_ALL(64);
    else if (E <= 128) MOE_ALL(128);
    else MOE_ALL(256);
#undef MOE_ALL
    return MOE_OK;
  }
  const int nv = (H + 511) / 512;
  if (T <= 64 && nv <= kFewMaxV) {
    switch (nv) {
#define MOE_FEW(NV)                                                                          \
  case NV:                                                                                   \
    MOE_LAUNCH(k_route_logits_few<NV>, dim3(E, (T + 15) / 16), dim3(256), 0, s, x, w_router, router_scale, \
               logit_bias, T, H, E, eps, logits, (int32_t *)nullptr, PrepArgs{});            \
    break;
      MOE_FEW(1) MOE_FEW(2) MOE_FEW(3) MOE_FEW(4) MOE_FEW(5) MOE_FEW(6) MOE_FEW(7)
      default: MOE_FEW(8)
#undef MOE_FEW
    }
  } else {
    const uint16_t *no_pes = nullptr;
    int32_t *no_idx = nullptr;
    float *no_w = nullptr;
    if (T < kWideExp16Below)
      MOE_LAUNCH((k_route_logits_wide<16, false>), dim3(E / 16, (T + kWideTok - 1) / kWideTok),
                 dim3(256), 0, s, x, w_router, router_scale, logit_bias, T, H, E, eps, logits,
                 no_pes, 0, no_idx, no_w, no_w, no_w, no_w);
    else
      MOE_LAUNCH((k_route_logits_wide<32, false>), dim3((E + 31) / 32, (T + kWideTok - 1) / kWideTok),
                 dim3(256), 0, s, x, w_router, router_scale, logit_bias, T, H, E, eps, logits,
                 no_pes, 0, no_idx, no_w, no_w, no_w, no_w);
  }
  MOE_LAUNCH(k_route_select, dim3((T + 3) / 4), dim3(256), 0, s, logits, per_expert_scale,
                     T, E, top_k, topk_idx, topk_w, topk_w_raw);
  return MOE_OK;
}

namespace moe {
namespace {
// the checks of moe_route and moe_bucket, before anything is queued
int route_bucket_checks(const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
                        const uint16_t *per_expert_scale, int32_t T, int32_t H, int32_t E,
                        int32_t top_k, int32_t *topk_idx, float *topk_w,
                        int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_rank,
                        void *workspace, size_t ws_bytes) {
  if (!w_router || !router_scale || !per_expert_scale || !expert_offsets || !workspace)
    return MOE_ERR_NULL;
  if (T > 0 && (!x || !topk_idx || !topk_w || !sorted_pairs || !pair_rank)) return MOE_ERR_NULL;
  if (T < 0 || H <= 0 || H % 64 || E <= 0 || top_k <= 0 || top_k > E) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS || E % 16 || top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  if (ws_bytes < moe_bucket_workspace_bytes(T, top_k, E)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// true: the decode path, logits (into the caller's buffer) then one
// selection + bucketing launch
bool fused_route(int T, int H, int top_k, const float *logits) {
  const int nv = (H + 511) / 512;
  return logits && T > 0 && T <= kFusedMaxT && nv <= kFewMaxV && T * top_k <= 4096;
}

// moe_route for many tokens with the logits split along K into ks slices,
// their partial sums in the moe_bucket workspace (arguments validated by the
// caller; ks <= route_split_ks(T, E), so the workspace holds them)
int route_split(const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
                 const uint16_t *per_expert_scale, const float *logit_bias, int32_t T, int32_t H,
                 int32_t E, int32_t top_k, float eps, int32_t *topk_idx, float *topk_w,
                 float *topk_w_raw, float *logits, int exp, int ks, void *workspace,
                 hipStream_t s) {
  float *part, *pss;
  route_partials(workspace, T, top_k, E, &part, &pss);
  const uint16_t *no_pes = nullptr;
  int32_t *no_idx = nullptr;
  float *no_w = nullptr;
#define MOE_SPLIT(EXP)                                                                         \
  MOE_LAUNCH((k_route_logits_wide<EXP, false, true>),                                          \
             dim3((E + EXP - 1) / EXP, (T + kWideTok - 1) / kWideTok, ks), dim3(256), 0, s, x,   \
             w_router, router_scale, logit_bias, T, H, E, eps, no_w, no_pes, 0, no_idx, no_w,   \
             no_w, part, pss)
  if (exp == 128) MOE_SPLIT(128);
  else if (exp == 64) MOE_SPLIT(64);
  else MOE_SPLIT(32);
#undef MOE_SPLIT
  if (E <= 2 * kWave)
    MOE_LAUNCH(k_route_select_split<2>, dim3((T + 3) / 4), dim3(256), 0, s, (const float *)part,
               (const float *)pss, ks, logit_bias, T, H, E, eps, logits, per_expert_scale, top_k,
               topk_idx, topk_w, topk_w_raw);
  else
    MOE_LAUNCH(k_route_select_split<MOE_MAX_EXPERTS / kWave>, dim3((T + 3) / 4), dim3(256), 0, s,
               (const float *)part, (const float *)pss, ks, logit_bias, T, H, E, eps, logits,
               per_expert_scale, top_k, topk_idx, topk_w, topk_w_raw);
  return MOE_OK;
}

int route_bucket_fused(const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
                       const uint16_t *per_expert_scale, const float *logit_bias, int32_t T,
                       int32_t H, int32_t E, int32_t top_k, float eps, int32_t *topk_idx,
                       float *topk_w, float *topk_w_raw, float *logits, int32_t *expert_offsets,
                       int32_t *sorted_pairs, int32_t *pair_rank, void *workspace,
                       const PrepArgs &pa, hipStream_t s) {
  const int nv = (H + 511) / 512;
  // the arrival counter of the selection kernel: word 1 of the workspace,
  // zeroed by the logits kernel of this call
  int32_t *arrive = (int32_t *)workspace + 1;
  switch (nv) {
#define MOE_FEW(NV)                                                                          \
  case NV:                                                                                   \
    MOE_LAUNCH(k_route_logits_few<NV>, dim3(E, (T + 15) / 16), dim3(256), 0, s, x, w_router, \
               router_scale, logit_bias, T, H, E, eps, logits, arrive, PrepArgs{});          \
    break;
    MOE_FEW(1) MOE_FEW(2) MOE_FEW(3) MOE_FEW(4) MOE_FEW(5) MOE_FEW(6) MOE_FEW(7)
    default: MOE_FEW(8)
#undef MOE_FEW
  }
  return launch_select_bucket(logits, per_expert_scale, T, E, top_k, topk_idx, topk_w, topk_w_raw,
                              expert_offsets, sorted_pairs, pair_rank, workspace, pa, s);
}
}  // namespace
}  // namespace moe

extern "C" int moe_route_bucket(const uint16_t *x, const uint16_t *w_router,
                                const uint16_t *router_scale, const uint16_t *per_expert_scale,
                                const float *logit_bias, int32_t T, int32_t H, int32_t E,
                                int32_t top_k, float eps, int32_t *topk_idx, float *topk_w,
                                float *topk_w_raw, float *logits, int32_t *expert_offsets,
                                int32_t *sorted_pairs, int32_t *pair_rank, void *workspace,
                                size_t ws_bytes, void *stream) {
  using namespace moe;
  int st = route_bucket_checks(x, w_router, router_scale, per_expert_scale, T, H, E, top_k,
                               topk_idx, topk_w, expert_offsets, sorted_pairs, pair_rank,
                               workspace, ws_bytes);
  if (st != MOE_OK) return st;
  if (!fused_route(T, H, top_k, logits)) {
    // T == 0 included: the offsets are all zero, as moe_bucket writes them
    int exp, ks;
    route_split_cfg(T, E, &exp, &ks);
    ks = min(ks, (H + kWideKC - 1) / kWideKC);
    if (ks > 0) {
      st = route_split(x, w_router, router_scale, per_expert_scale, logit_bias, T, H, E, top_k, eps,
                       topk_idx, topk_w, topk_w_raw, logits, exp, ks, workspace, (hipStream_t)stream);
      if (st != MOE_OK) return st;
    } else if (T > 0) {
      st = moe_route(x, w_router, router_scale, per_expert_scale, logit_bias, T, H, E, top_k,
                     eps, topk_idx, topk_w, topk_w_raw, logits, stream);
      if (st != MOE_OK) return st;
    }
    return moe_bucket(topk_idx, T, top_k, E, expert_offsets, sorted_pairs, pair_rank, workspace,
                      ws_bytes, stream);
  }
  return route_bucket_fused(x, w_router, router_scale, per_expert_scale, logit_bias, T, H, E,
                            top_k, eps, topk_idx, topk_w, topk_w_raw, logits, expert_offsets,
                            sorted_pairs, pair_rank, workspace, PrepArgs{}, (hipStream_t)stream);
}

extern "C" int moe_route_bucket_prep(
    const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
    const uint16_t *per_expert_scale, const float *logit_bias, int32_t T, int32_t H, int32_t E,
    int32_t top_k, float eps, int32_t *topk_idx, float *topk_w, float *topk_w_raw, float *logits,
    int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_rank, void *bucket_ws,
    size_t bucket_ws_bytes, const uint16_t *norm_weight, float norm_eps, int32_t I,
    void *expert_ws, size_t expert_ws_bytes, void *stream) {
  using namespace moe;
  int st = route_bucket_checks(x, w_router, router_scale, per_expert_scale, T, H, E, top_k,
                               topk_idx, topk_w, expert_offsets, sorted_pairs, pair_rank,
                               bucket_ws, bucket_ws_bytes);
  if (st != MOE_OK) return st;
  if (norm_weight && !(norm_eps >= 0.0f)) return MOE_ERR_SHAPE;
  PrepArgs pa{};
  st = expert_prep_buffers(T, top_k, E, H, I, expert_ws, expert_ws_bytes, &pa.x16, &pa.x_exp,
                           &pa.a_max);
  if (st != MOE_OK) return st;
  if (!fused_route(T, H, top_k, logits)) {
    st = moe_route_bucket(x, w_router, router_scale, per_expert_scale, logit_bias, T, H, E, top_k,
                          eps, topk_idx, topk_w, topk_w_raw, logits, expert_offsets, sorted_pairs,
                          pair_rank, bucket_ws, bucket_ws_bytes, stream);
    if (st != MOE_OK) return st;
    return norm_weight ? nvfp4_expert_prep_rmsnorm(x, norm_weight, norm_eps, T, top_k, E, H, I,
                                                   expert_ws, expert_ws_bytes, stream)
                       : nvfp4_expert_prep(x, T, top_k, E, H, I, expert_ws, expert_ws_bytes,
                                           stream);
  }
  pa.x = x;
  pa.norm_w = norm_weight;
  pa.norm_eps = norm_eps;
  pa.H = H;
  pa.P = T * top_k;
  return route_bucket_fused(x, w_router, router_scale, per_expert_scale, logit_bias, T, H, E,
                            top_k, eps, topk_idx, topk_w, topk_w_raw, logits, expert_offsets,
                            sorted_pairs, pair_rank, bucket_ws, pa, (hipStream_t)stream);
}

namespace moe {
// The fused decode layer's first kernel: the router logits of T <= 64 tokens
// (H <= 4096) into `logits`, beside the expert input's prep (pa) in
// ceil(T/4) more workgroups.  Arguments validated by the caller.
__attribute__((visibility("hidden"))) int launch_route_logits_prep(
    const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
    const float *logit_bias, int T, int H, int E, float eps, float *logits, const PrepArgs &pa,
    hipStream_t s) {
  const int nv = (H + 511) / 512;
  const dim3 grid(E + (T + 3) / 4, (T + 15) / 16);
  switch (nv) {
#define MOE_FEW(NV)                                                                          \
  case NV:                                                                                   \
    MOE_LAUNCH(k_route_logits_few<NV>, grid, dim3(256), 0, s, x, w_router, router_scale,      \
               logit_bias, T, H, E, eps, logits, (int32_t *)nullptr, pa);                    \
    break;
    MOE_FEW(1) MOE_FEW(2) MOE_FEW(3) MOE_FEW(4) MOE_FEW(5) MOE_FEW(6) MOE_FEW(7)
    default: MOE_FEW(8)
#undef MOE_FEW
  }
  return MOE_OK;
}
}  // namespace moe
