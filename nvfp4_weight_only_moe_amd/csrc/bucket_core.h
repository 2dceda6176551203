// Pieces of the stable sort of (token, slot) pairs by expert shared by the
// bucketing kernels and the fused decode layer ("Gemma 4 26B-A4B (MoE) - Core
// AI", Decode only: the sort-by-expert step of a grouped GEMM).  Order is
// (expert, pair id p = t * top_k + j); ids outside [0, E) form a bucket E
// after every expert, are counted, and get rank -1.
#pragma once
#include "common.h"

namespace moe {

constexpr int kMaxB = MOE_MAX_EXPERTS + 1;  // buckets incl. the invalid one

__device__ __forceinline__ int bucket_of(int e, int E) { return (e >= 0 && e < E) ? e : E; }

// Exclusive scan of cnt[0..nb) into out[0..nb) by the first wave (nb <= 257).
__device__ __forceinline__ void wave_exclusive_scan(const int *cnt, int *out, int nb) {
  const int lane = threadIdx.x;
  if (lane >= kWave) return;
  int carry = 0;
  for (int base = 0; base < nb; base += kWave) {
    const int i = base + lane;
    int v = i < nb ? cnt[i] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    if (i < nb) out[i] = carry + incl - v;
    carry += __shfl(incl, kWave - 1, kWave);
  }
}

// The whole bucketing of P <= 64 pairs by the first wave of a workgroup (lane
// p holds pair p): offsets [E+1] (in LDS: read back here), sorted [P] and
// rank [P] (LDS or memory), *err = the number of invalid ids.  s_cnt: LDS for
// E + 1 ints.  Counts by ballots, offsets by one DPP prefix sum (lane l holds
// experts 4l .. 4l + 3).  No barrier: the caller synchronises before other
// waves read the results.
__device__ __forceinline__ void bucket_one_wave(const int32_t *idx, int P, int E, int32_t *offsets,
                                                int32_t *sorted, int32_t *rank, int32_t *err,
                                                int *s_cnt) {
  constexpr int PER = MOE_MAX_EXPERTS / kWave;  // 4
  const int lane = threadIdx.x;
  if (lane >= kWave) return;
  for (int i = lane; i <= E; i += kWave) s_cnt[i] = 0;
  const bool valid = lane < P;
  const int b = valid ? bucket_of(idx[lane], E) : 0;
  // lanes holding the same bucket: 9 ballots over the bits of b (nb <= 257)
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {
    const bool on = (b >> bit) & 1;
    const unsigned long long m = __ballot(on);
    peers &= on ? m : ~m;
  }
  const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int before = __popcll(peers & lt);           // same bucket, lower pair id
  if (valid && before == 0) s_cnt[b] = __popcll(peers);
  __builtin_amdgcn_wave_barrier();
  int c[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = PER * lane + i < E ? s_cnt[PER * lane + i] : 0;
    sum += c[i];
  }
  const int incl = wave_incl_scan(sum);
  int base = incl - sum;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (PER * lane + i < E) offsets[PER * lane + i] = base;
    base += c[i];
  }
  const int nvalid = __builtin_amdgcn_readlane(incl, kWave - 1);  // bucket E starts here
  if (lane == 0) {
    offsets[E] = nvalid;
    *err = s_cnt[E];
  }
  __builtin_amdgcn_wave_barrier();
  if (valid) {
    const int pos = (b == E ? nvalid : offsets[b]) + before;
    sorted[pos] = lane;
    rank[lane] = b == E ? -1 : pos;
  }
}

}  // namespace moe
