// moe_bucket: stable counting sort of the (token, slot) pairs by expert -- the
// sort-by-expert step of a grouped GEMM ("Gemma 4 26B-A4B (MoE) - Core AI",
// Decode only: batched sort-by-expert kernel for more than one token).
//
// Order is (expert, token, slot), i.e. by expert and then by pair id
// p = t*top_k + j.  Pairs with an id outside [0, E) go to an extra bucket E
// placed after all experts, are counted in the error word and get rank -1
// (so the combine adds nothing for them).
//
// Up to kSmallP pairs: one workgroup does everything (LDS histogram, scan,
// stable scatter).  Beyond that, in chunks of kChunk pairs: (1) per-chunk
// LDS histograms, (2) one
// workgroup turns them into expert offsets and per-chunk base positions,
// (3) per-chunk stable scatter.  The in-chunk rank of a pair among pairs of the
// same expert comes from a wave "multi-split": 9 ballots give each lane the
// mask of lanes holding the same bucket; a popcount below the lane is its rank
// in the wave, per-wave counts in LDS order the waves.  No atomics decide any
// position, so the output is the same on every run.
#include "bucket_core.h"
#include "common.h"
#include "select.h"

namespace moe {
namespace {

constexpr int kBucketThreads = 256;
constexpr int kBucketWaves = kBucketThreads / kWave;
constexpr int kSmallP = 4096;            // up to this many pairs: one workgroup
constexpr int kChunk = 1024;             // pairs per workgroup beyond that


// Stable scatter of the n bucket ids in s_b (pairs pbase .. pbase+n-1),
// starting from the per-bucket positions in s_run (updated in place), by a
// workgroup of THREADS threads.
template <int THREADS = kBucketThreads>
__device__ void scatter_rounds(const int *s_b, int n, int pbase, int nb, int *s_run,
                               int (*s_wcnt)[kMaxB], int32_t *sorted, int32_t *rank) {
  constexpr int WAVES = THREADS / kWave;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const unsigned long long lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int base = 0; base < n; base += THREADS) {
    const int i = base + tid;
    const bool valid = i < n;
    const int b = valid ? s_b[i] : 0;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
      const bool on = (b >> bit) & 1;
      const unsigned long long m = __ballot(on);
      peers &= on ? m : ~m;
    }
    const int rank_w = __popcll(peers & lt);
    if (valid && rank_w == 0) s_wcnt[wave][b] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = s_run[b];
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][b];
      pos += rank_w;
      const int p = pbase + i;
      sorted[pos] = p;
      rank[p] = b == nb - 1 ? -1 : pos;  // the invalid bucket: no rank, no expert
    }
    __syncthreads();
    for (int bb = tid; bb < nb; bb += THREADS) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        s += s_wcnt[w][bb];
        s_wcnt[w][bb] = 0;
      }
      s_run[bb] += s;
    }
    __syncthreads();
  }
}

template <int THREADS = kBucketThreads>
__device__ void zero_wcnt(int (*s_wcnt)[kMaxB], int nb) {
  for (int i = threadIdx.x; i < THREADS / kWave * nb; i += THREADS) s_wcnt[i / nb][i % nb] = 0;
}

// Every step of the bucketing for P <= kSmallP pairs by one workgroup of
// THREADS threads: LDS histogram, scan, stable scatter.
template <int THREADS>
__device__ __forceinline__ void bucket_small(const int32_t *__restrict__ idx, int P, int E,
                                             int32_t *__restrict__ offsets,
                                             int32_t *__restrict__ sorted,
                                             int32_t *__restrict__ rank, int32_t *__restrict__ err) {
  __shared__ int s_b[kSmallP];
  __shared__ int s_cnt[kMaxB], s_run[kMaxB];
  __shared__ int s_wcnt[THREADS / kWave][kMaxB];
  const int tid = threadIdx.x, nb = E + 1;
  for (int i = tid; i < nb; i += THREADS) s_cnt[i] = 0;
  zero_wcnt<THREADS>(s_wcnt, nb);
  __syncthreads();
  for (int p = tid; p < P; p += THREADS) {
    const int b = bucket_of(idx[p], E);
    s_b[p] = b;
    atomicAdd(&s_cnt[b], 1);
  }
  __syncthreads();
  wave_exclusive_scan(s_cnt, s_run, nb);
  __syncthreads();
  for (int i = tid; i < nb; i += THREADS) offsets[i] = s_run[i];
  if (tid == 0) err[0] = s_cnt[E];
  __syncthreads();
  scatter_rounds<THREADS>(s_b, P, 0, nb, s_run, s_wcnt, sorted, rank);
}

__global__ __launch_bounds__(kBucketThreads) void k_bucket_small(const int32_t *__restrict__ idx,
                                                                 int P, int E,
                                                                 int32_t *__restrict__ offsets,
                                                                 int32_t *__restrict__ sorted,
                                                                 int32_t *__restrict__ rank,
                                                                 int32_t *__restrict__ err) {
  bucket_small<kBucketThreads>(idx, P, E, offsets, sorted, rank, err);
}

// Selection over many workgroups (a wave per token, 4 tokens per workgroup),
// then the bucketing by the workgroup that finishes last: after its writes a
// workgroup takes one release fence and increments the arrival counter
// (zeroed by the logits kernel queued just before); the one that sees the
// final count takes an acquire fence and buckets every pair.  No workgroup
// waits for another.
__global__ __launch_bounds__(kBucketThreads) void k_select_bucket_last(
    const float *__restrict__ logits, const uint16_t *__restrict__ pes, int T, int E, int K,
    int32_t *topk_idx, float *__restrict__ topk_w, float *__restrict__ topk_w_raw,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted, int32_t *__restrict__ rank,
    int32_t *__restrict__ err, int32_t *__restrict__ arrive, PrepArgs pa) {
  __shared__ int s_arr;
  constexpr int kTPB = kBucketThreads / kWave;  // tokens per workgroup (a wave each)
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kTPB + wave;
  if (t < T) select_token(logits, pes, t, E, K, topk_idx, topk_w, topk_w_raw);
  __syncthreads();  // every wave's stores have left for L2
  if (threadIdx.x == 0) {
    __threadfence();  // release: this workgroup's selections, visible device-wide
    const int arr = atomicAdd(arrive, 1);
    if (arr == (int)gridDim.x - 1) __threadfence();  // acquire: every workgroup's selections
    s_arr = arr;
  }
  __syncthreads();
  const int arr = s_arr, G = (int)gridDim.x;
  const bool last = arr == G - 1;  // uniform
  if (last) bucket_small<kBucketThreads>(topk_idx, T * K, E, offsets, sorted, rank, err);
  // the expert-input prep (moe_route_bucket_prep) by arrival order: the
  // workgroup that arrived a-th preps token block a, except that the last one
  // (busy bucketing, on the critical path) leaves its block to the first one;
  // a single workgroup does both, bucketing first
  if (pa.x16) {
    for (int i = blockIdx.x * kBucketThreads + threadIdx.x; i < pa.P; i += G * kBucketThreads)
      pa.a_max[i] = 0u;
    auto prep_block = [&](int blk) {
      const int tp = blk * kTPB + wave;
      if (tp >= T) return;
      if (pa.norm_w)
        prep_row<true>(pa.x, pa.norm_w, pa.norm_eps, pa.H, tp, pa.x16, pa.x_exp);
      else
        prep_row<false>(pa.x, nullptr, 0.0f, pa.H, tp, pa.x16, pa.x_exp);
    };
    if (!last || G == 1) prep_block(arr);
    if (arr == 0 && G > 1) prep_block(G - 1);
  }
}

__global__ __launch_bounds__(kBucketThreads) void k_bucket_hist(const int32_t *__restrict__ idx,
                                                                int P, int E,
                                                                int32_t *__restrict__ chunk_cnt) {
  __shared__ int s_cnt[kMaxB];
  const int tid = threadIdx.x, nb = E + 1, c = blockIdx.x;
  for (int i = tid; i < nb; i += kBucketThreads) s_cnt[i] = 0;
  __syncthreads();
  const int p0 = c * kChunk, p1 = min(P, p0 + kChunk);
  for (int p = p0 + tid; p < p1; p += kBucketThreads) atomicAdd(&s_cnt[bucket_of(idx[p], E)], 1);
  __syncthreads();
  for (int i = tid; i < nb; i += kBucketThreads) chunk_cnt[(size_t)c * nb + i] = s_cnt[i];
}

__global__ __launch_bounds__(kBucketThreads) void k_bucket_scan(const int32_t *__restrict__ chunk_cnt,
                                                                int nchunks, int E,
                                                                int32_t *__restrict__ chunk_base,
                                                                int32_t *__restrict__ offsets,
                                                                int32_t *__restrict__ err) {
  __shared__ int s_tot[kMaxB], s_off[kMaxB];
  const int tid = threadIdx.x, nb = E + 1;
  // the chunk loops are unrolled so that many independent count loads are
  // in flight at once (the sums themselves stay in chunk order)
  for (int b = tid; b < nb; b += kBucketThreads) {
    int s = 0;
#pragma unroll 16
    for (int c = 0; c < nchunks; ++c) s += chunk_cnt[(size_t)c * nb + b];
    s_tot[b] = s;
  }
  __syncthreads();
  wave_exclusive_scan(s_tot, s_off, nb);
  __syncthreads();
  for (int b = tid; b < nb; b += kBucketThreads) {
    offsets[b] = s_off[b];
    int run = s_off[b];
#pragma unroll 16
    for (int c = 0; c < nchunks; ++c) {
      chunk_base[(size_t)c * nb + b] = run;
      run += chunk_cnt[(size_t)c * nb + b];
    }
  }
  if (tid == 0) err[0] = s_tot[E];
}

__global__ __launch_bounds__(kBucketThreads) void k_bucket_scatter(
    const int32_t *__restrict__ idx, int P, int E, const int32_t *__restrict__ chunk_base,
    int32_t *__restrict__ sorted, int32_t *__restrict__ rank) {
  __shared__ int s_b[kChunk];
  __shared__ int s_run[kMaxB];
  __shared__ int s_wcnt[kBucketWaves][kMaxB];
  const int tid = threadIdx.x, nb = E + 1, c = blockIdx.x;
  const int p0 = c * kChunk, n = min(P, p0 + kChunk) - p0;
  for (int i = tid; i < nb; i += kBucketThreads) s_run[i] = chunk_base[(size_t)c * nb + i];
  zero_wcnt<kBucketThreads>(s_wcnt, nb);
  for (int i = tid; i < n; i += kBucketThreads) s_b[i] = bucket_of(idx[p0 + i], E);
  __syncthreads();
  scatter_rounds<kBucketThreads>(s_b, n, p0, nb, s_run, s_wcnt, sorted, rank);
}

// Workspace: error word and arrival counter, per-chunk bucket counts and
// bases, then (for moe_route_bucket with K-split router logits) the router's
// partial dot products [ks][T][E] and partial sums of squares [ks][T].
size_t bucket_ws_layout(int T, int top_k, int E, size_t *cnt_off, size_t *base_off,
                        size_t *route_off = nullptr) {
  const size_t P = (size_t)T * top_k;
  const size_t nchunks = (P + kChunk - 1) / kChunk;
  const size_t nb = (size_t)E + 1;
  *cnt_off = 256;
  *base_off = *cnt_off + moe_align_up(nchunks * nb * 4, 256);
  const size_t ro = *base_off + moe_align_up(nchunks * nb * 4, 256);
  if (route_off) *route_off = ro;
  const size_t ks = (size_t)route_split_ks(T, E);
  return ro + (ks > 0 ? moe_align_up(ks * T * E * 4, 256) + moe_align_up(ks * T * 4, 256) : 0);
}

}  // namespace
}  // namespace moe

namespace moe {
// The K-split router's partial buffers in a moe_bucket workspace (valid when
// route_split_ks(T, E) > 0).
__attribute__((visibility("hidden"))) void route_partials(void *workspace, int T, int top_k, int E,
                                                          float **part, float **pss) {
  size_t a, b, ro;
  bucket_ws_layout(T, top_k, E, &a, &b, &ro);
  const int ks = route_split_ks(T, E);
  *part = (float *)((char *)workspace + ro);
  *pss = (float *)((char *)workspace + ro + moe_align_up((size_t)ks * T * E * 4, 256));
}
}  // namespace moe

namespace moe {
// Selection + bucketing in one launch for T tokens with T * top_k <= kSmallP
// (arguments validated by the caller, moe_route_bucket); the arrival counter
// is word 1 of the workspace, zeroed by the logits kernel queued before.
__attribute__((visibility("hidden"))) int launch_select_bucket(
                         const float *logits, const uint16_t *pes, int T, int E, int top_k,
                         int32_t *topk_idx, float *topk_w, float *topk_w_raw,
                         int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_rank,
                         void *workspace, const PrepArgs &pa, hipStream_t s) {
  int32_t *err = (int32_t *)workspace;
  MOE_LAUNCH(k_select_bucket_last, dim3((T + kBucketWaves - 1) / kBucketWaves),
             dim3(kBucketThreads), 0, s, logits, pes, T, E, top_k, topk_idx, topk_w, topk_w_raw,
             expert_offsets, sorted_pairs, pair_rank, err, err + 1, pa);
  return MOE_OK;
}
}  // namespace moe

extern "C" size_t moe_bucket_workspace_bytes(int32_t T, int32_t top_k, int32_t E) {
  if (T < 0 || top_k <= 0 || E <= 0) return 0;
  size_t a, b;
  return moe::bucket_ws_layout(T, top_k, E, &a, &b);
}

extern "C" int moe_bucket(const int32_t *topk_idx, int32_t T, int32_t top_k, int32_t E,
                          int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_rank,
                          void *workspace, size_t ws_bytes, void *stream) {
  using namespace moe;
  if (!expert_offsets || !workspace || (T > 0 && (!topk_idx || !sorted_pairs || !pair_rank)))
    return MOE_ERR_NULL;
  if (T < 0 || top_k <= 0 || E <= 0) return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  size_t cnt_off, base_off;
  const size_t need = bucket_ws_layout(T, top_k, E, &cnt_off, &base_off);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int P = T * top_k;
  int32_t *err = (int32_t *)workspace;
  if (P <= kSmallP) {
    MOE_LAUNCH(k_bucket_small, dim3(1), dim3(kBucketThreads), 0, s, topk_idx, P, E,
                       expert_offsets, sorted_pairs, pair_rank, err);
    return MOE_OK;
  }
  const int nchunks = (P + kChunk - 1) / kChunk;
  int32_t *chunk_cnt = (int32_t *)((char *)workspace + cnt_off);
  int32_t *chunk_base = (int32_t *)((char *)workspace + base_off);
  MOE_LAUNCH(k_bucket_hist, dim3(nchunks), dim3(kBucketThreads), 0, s, topk_idx, P, E,
                     chunk_cnt);
  MOE_LAUNCH(k_bucket_scan, dim3(1), dim3(kBucketThreads), 0, s, chunk_cnt, nchunks, E,
                     chunk_base, expert_offsets, err);
  MOE_LAUNCH(k_bucket_scatter, dim3(nchunks), dim3(kBucketThreads), 0, s, topk_idx, P, E,
                     chunk_base, sorted_pairs, pair_rank);
  return MOE_OK;
}
