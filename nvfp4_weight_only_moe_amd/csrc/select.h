// Top-k selection of one token, shared by the router's selection kernel and
// the fused selection + bucketing kernel ("Gemma 4 26B-A4B (MoE) - Core AI",
// Architecture, router description: softmax over all experts in fp32, top-k,
// renormalise to sum 1, times per_expert_scale at the chosen ids).
#pragma once
#include "common.h"

namespace moe {

// Cross-lane steps of the selection: DPP moves within 16-lane rows (xor 1,
// xor 2, half-row mirror, row mirror) leave every lane of a row holding the
// row's result; four lane reads combine the rows into a wave-uniform value.
// Each step has a few cycles of latency, where an LDS permute has tens.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, dpp_mov<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ float lane_read(float v, int lane) {
  return __builtin_bit_cast(float, lane_read(__builtin_bit_cast(uint32_t, v), lane));
}
// wave maximum of unsigned keys -> uniform (exact in any order)
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
  v = max(v, dpp_mov<0xB1>(v));
  v = max(v, dpp_mov<0x4E>(v));
  v = max(v, dpp_mov<0x141>(v));
  v = max(v, dpp_mov<0x140>(v));
  return max(max(lane_read(v, 0), lane_read(v, 16)), max(lane_read(v, 32), lane_read(v, 48)));
}
// wave sum in a fixed order (the same in every lane) -> uniform
__device__ __forceinline__ float wave_sum_u(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

// Order-preserving map of a float to an unsigned key (larger float, larger
// key; -inf -> 0x007FFFFF); key 0 marks an expert that is not a candidate.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// One wave selects for token t from logits[t][0..E): softmax over all E in
// fp32, k rounds of selecting the largest remaining logit (ties to the lower
// expert id), renormalisation over the k chosen probabilities, times
// per_expert_scale at the chosen ids.  Lane l holds experts l, l + 64, ...
// (NPER of them, 64 NPER >= E).  A NaN logit is treated as -inf, so every
// round finds a candidate and the ids are always distinct and in [0, E).
// The logits row `lrow` (E floats) is in global memory (buffer loads), or in
// LDS when LDS is true.
template <int NPER, bool LDS = false>
__device__ __forceinline__ void select_token_n(const float *__restrict__ lrow,
                                               const uint16_t *__restrict__ pes, int t, int E,
                                               int K, int32_t *__restrict__ topk_idx,
                                               float *__restrict__ topk_w,
                                               float *__restrict__ topk_w_raw) {
  const int lane = threadIdx.x & 63;
  t = __builtin_amdgcn_readfirstlane(t);  // one token per wave: uniform
  // unguarded buffer loads (lanes past E read zeros), all in flight at once;
  // per_expert_scale of this lane's experts is loaded up front as well
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(pes, (uint32_t)E * 2u);
  uint32_t lraw[NPER], praw[NPER];
  if (LDS) {
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = lane + i * kWave;
      lraw[i] = e < E ? __float_as_uint(lrow[e]) : 0u;
      praw[i] = bload2(rp, (uint32_t)e * 2u);
    }
  } else {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(lrow, (uint32_t)E * 4u);
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const uint32_t e = lane + i * kWave;
      lraw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rl, e * 4u, 0, 0);
      praw[i] = bload2(rp, e * 2u);
    }
  }
  float v[NPER];
  uint32_t key[NPER];
  uint32_t kmax = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const float x = __uint_as_float(lraw[i]);
    const bool ok = lane + i * kWave < E;
    v[i] = (ok && x == x) ? x : -__builtin_huge_valf();
    key[i] = ok ? float_key(v[i]) : 0u;
    kmax = max(kmax, key[i]);
  }
  const float m = key_float(wave_max_key(kmax));
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < NPER; ++i) z += (lane + i * kWave < E) ? expf(v[i] - m) : 0.0f;
  z = wave_sum_u(z);

  // round s: the largest remaining key; lane s keeps its id, key and scale
  uint32_t my_id = 0, my_key = 0, my_pes = 0;
  for (int s = 0; s < K; ++s) {
    uint32_t b = key[0];
#pragma unroll
    for (int i = 1; i < NPER; ++i) b = max(b, key[i]);
    const uint32_t ms = wave_max_key(b);
    // lowest id holding ms: the first item index with a match, then the
    // lowest matching lane
    int id = 0;
    uint32_t pw = 0;
#pragma unroll
    for (int i = NPER - 1; i >= 0; --i) {
      const unsigned long long hit = __ballot(key[i] == ms);
      if (hit) {
        const int l = (int)__builtin_ctzll(hit);
        id = i * kWave + l;
        pw = lane_read(praw[i], l);
      }
    }
    id = __builtin_amdgcn_readfirstlane(id);
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (lane + i * kWave == id) key[i] = 0u;
    if (lane == s) {
      my_id = (uint32_t)id;
      my_key = ms;
      my_pes = pw;
    }
  }
  // probabilities of the k selections (lane s: selection s), their sum in a
  // fixed order, and the renormalised weights
  const float p = lane < K ? expf(key_float(my_key) - m) / z : 0.0f;
  const float psum = wave_sum_u(p);
  if (lane < K) {
    const float wr = p / psum;
    topk_idx[(size_t)t * K + lane] = (int32_t)my_id;
    topk_w[(size_t)t * K + lane] = wr * bf16_to_f32((uint16_t)my_pes);
    if (topk_w_raw) topk_w_raw[(size_t)t * K + lane] = wr;
  }
}

// NT tokens by one wave at once (t0, t0 + tstride, ...; those at or past T
// are skipped): the same arithmetic as select_token_n, token by token, with
// the NT independent chains of each round interleaved so that their
// cross-lane latencies overlap.
template <int NPER, int NT>
__device__ __forceinline__ void select_tokens_n(const float *__restrict__ logits,
                                                const uint16_t *__restrict__ pes, int t0,
                                                int tstride, int T, int E, int K,
                                                int32_t *__restrict__ topk_idx,
                                                float *__restrict__ topk_w,
                                                float *__restrict__ topk_w_raw) {
  const int lane = threadIdx.x & 63;
  t0 = __builtin_amdgcn_readfirstlane(t0);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(pes, (uint32_t)E * 2u);
  uint32_t praw[NPER];
  uint32_t key[NT][NPER];
  float v[NT][NPER];
  bool on[NT];
#pragma unroll
  for (int i = 0; i < NPER; ++i) praw[i] = bload2(rp, (uint32_t)(lane + i * kWave) * 2u);
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const int t = t0 + q * tstride;
    on[q] = t < T;
    const __amdgpu_buffer_rsrc_t rl =
        make_rsrc(logits + (size_t)(on[q] ? t : 0) * E, on[q] ? (uint32_t)E * 4u : 0u);
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const uint32_t x = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)(lane + i * kWave) * 4u, 0, 0);
      const float f = __uint_as_float(x);
      const bool ok = lane + i * kWave < E;
      v[q][i] = (ok && f == f) ? f : -__builtin_huge_valf();
      key[q][i] = ok ? float_key(v[q][i]) : 0u;
    }
  }
  float m[NT], z[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    uint32_t kmax = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) kmax = max(kmax, key[q][i]);
    m[q] = key_float(wave_max_key(kmax));
  }
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    float zz = 0.0f;
#pragma unroll
    for (int i = 0; i < NPER; ++i) zz += (lane + i * kWave < E) ? expf(v[q][i] - m[q]) : 0.0f;
    z[q] = wave_sum_u(zz);
  }
  uint32_t my_id[NT], my_key[NT], my_pes[NT];
#pragma unroll
  for (int q = 0; q < NT; ++q) my_id[q] = my_key[q] = my_pes[q] = 0;
  for (int s = 0; s < K; ++s) {
    uint32_t ms[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      uint32_t b = key[q][0];
#pragma unroll
      for (int i = 1; i < NPER; ++i) b = max(b, key[q][i]);
      ms[q] = wave_max_key(b);
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      int id = 0;
      uint32_t pw = 0;
#pragma unroll
      for (int i = NPER - 1; i >= 0; --i) {
        const unsigned long long hit = __ballot(key[q][i] == ms[q]);
        if (hit) {
          const int l = (int)__builtin_ctzll(hit);
          id = i * kWave + l;
          pw = lane_read(praw[i], l);
        }
      }
      id = __builtin_amdgcn_readfirstlane(id);
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (lane + i * kWave == id) key[q][i] = 0u;
      if (lane == s) {
        my_id[q] = (uint32_t)id;
        my_key[q] = ms[q];
        my_pes[q] = pw;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const float p = lane < K ? expf(key_float(my_key[q]) - m[q]) / z[q] : 0.0f;
    const float psum = wave_sum_u(p);
    const int t = t0 + q * tstride;
    if (on[q] && lane < K) {
      const float wr = p / psum;
      topk_idx[(size_t)t * K + lane] = (int32_t)my_id[q];
      topk_w[(size_t)t * K + lane] = wr * bf16_to_f32((uint16_t)my_pes[q]);
      if (topk_w_raw) topk_w_raw[(size_t)t * K + lane] = wr;
    }
  }
}

__device__ __forceinline__ void select_token(const float *__restrict__ logits,
                                             const uint16_t *__restrict__ pes, int t, int E,
                                             int K, int32_t *__restrict__ topk_idx,
                                             float *__restrict__ topk_w,
                                             float *__restrict__ topk_w_raw) {
  if (E <= 2 * kWave)
    select_token_n<2>(logits + (size_t)t * E, pes, t, E, K, topk_idx, topk_w, topk_w_raw);
  else
    select_token_n<MOE_MAX_EXPERTS / kWave>(logits + (size_t)t * E, pes, t, E, K, topk_idx, topk_w,
                                            topk_w_raw);
}

}  // namespace moe
