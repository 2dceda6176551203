// nvfp4_expert_mlp: the routed experts of the Gemma-4 MoE block on gfx950.
//
// Per expert e and its bucket of rows X_e ("Gemma 4 26B-A4B (MoE) - Core AI",
// Architecture: GELU-gated experts, gelu_pytorch_tanh; gate/up 2816 -> 704,
// down 704 -> 2816):
//     A = gelu_tanh(X_e Wg^T) * (X_e Wu^T),   Y = A Wd^T
// with W = E2M1 x E4M3 block scale x FP32 tensor scale ("Gemma-4-26B-A4B-
// NVFP4-mlx", Notes).
//
// Stages (also public entry points):
//  * prep: per token, the exponent of max|x| and the f16 copy of the row
//    scaled by 2^(14 - exponent) (exact for every bf16 value down to 2^-29 of
//    the row maximum), in token order -- it does not depend on the routing, so
//    a caller can run it beside moe_route / moe_bucket; clears the per-row
//    maximum of A.
//  * gate/up and down: grouped GEMMs over (expert, row-block) tiles; each
//    workgroup finds its tile from expert_offsets with one wave-wide scan.
//    Weights are read in the tiled layout (one contiguous kilobyte per wave
//    load, already in matrix-core operand order) through buffer resources
//    (lanes past K read hardware zeros) and dequantised in registers: hardware
//    FP4 -> f16 conversion times the E4M3 block scale in f16 (exact), then f16
//    MFMAs 16x16x32 with fp32 accumulation.  The tensor scale and the row's
//    power of two are applied to the fp32 sums.
//    Two kernel families, chosen from host-known shapes only:
//     - GEMV mode (few rows per expert, decode): every wave is an independent
//       stream, no LDS staging and no barrier in the K loop; each lane loads
//       its activation chunks (16 bytes of one row, row-major [row][K]) with
//       buffer loads straight into MFMA operand registers.
//     - tiled mode (prefill): 16*MSUB rows per tile staged in LDS per K unit
//       and shared by the 4 waves, weights streamed once per tile; 64-row
//       tiles, or 128-row tiles once buckets average 192 rows (their
//       accumulators held in place in the accumulation registers; down then
//       reads A converted once to row-scaled f16).
//    Gate/up epilogue: GELU-tanh gating, A rounded to bf16 (row-major
//    [P][I] in sorted-row order), per-row max|A| by atomicMax on the float
//    bits (an integer max: order-independent).  Down rescales A to f16 by that maximum's power
//    of two and writes Y as bf16 in sorted-row order.
#include <mutex>
#include <type_traits>

#include "bucket_core.h"
#include "common.h"
#include "select.h"

namespace moe {
namespace {

constexpr int kBM = 16;        // rows per tile (one MFMA M)
constexpr int kCols = 64;      // output columns per workgroup (4 waves x 16)
constexpr int kThreads = 256;

struct Nvfp4 {
  const uint8_t *packed;
  const uint8_t *scales;
  const float *global;
};

struct WsLayout {
  size_t x_exp, a_max, x16, a, a16, total;
  int max_tiles;
};

// rows per tile: 16 x MSUB, from the mean bucket size (host-known shapes
// only).  MSUB = 1 selects GEMV mode.
int choose_msub(int T, int top_k, int E) {
  const long long P = (long long)T * top_k;
  const long long buckets = P < E ? P : E;
  const long long avg = buckets > 0 ? P / buckets : 0;
  if (avg < 24) return 1;
  return 4;
}

// rows per expert-GEMM block in tiled mode: 128 (MSUB = 8) once buckets hold
// 128 rows or more on average, else 64.  Measured against 64-row blocks at
// 2048 tokens (128 rows per expert on average): gate/up 198 -> 176 us with
// Zipf routing, 199 -> 179 us with uniform routing; 4-15% faster from 256
// rows up.  (Before the gate/up blocks were spread over the XCDs by cost,
// the crossover lay near 192 rows.)
constexpr int kMsub8From = 128;
// (and the expert intermediate I fits the row conversion of the down
// blocks, k_a_f16: at most 4096)
int gate_up_msub(int T, int top_k, int E, int I) {
  const int m = choose_msub(T, top_k, E);
  if (m == 1) return 1;
  const long long P = (long long)T * top_k;
  const long long buckets = P < E ? P : E;
  return P / buckets >= kMsub8From && I <= 4096 ? 8 : m;
}

// Few rows per expert (decode): the GEMV-mode kernels.  Otherwise tiled mode.
bool gemv_mode(int T, int top_k, int E) { return choose_msub(T, top_k, E) == 1; }

// rows per tile in GEMV mode: 8 for up to 4 rows per expert on average, else 16
int gemv_rows(int T, int top_k, int E) { return (long long)T * top_k <= 4LL * E ? 8 : 16; }

// rows per tile of the expert kernels
int tile_rows(int T, int top_k, int E) {
  return gemv_mode(T, top_k, E) ? gemv_rows(T, top_k, E) : kBM * choose_msub(T, top_k, E);
}

// Workspace: token exponents [T], per-row max of A [P], the f16 activations
// [T][H], A [P][I] bf16 (and, with 128-row blocks, A [P][I] as f16 scaled by
// its row's power of two).  max_tiles bounds the tile count (sum over experts
// of ceil(M_e / rows)) for the grids.
WsLayout ws_layout(int T, int top_k, int E, int H, int I) {
  WsLayout L;
  const size_t P = (size_t)T * top_k;
  const int bm = tile_rows(T, top_k, E);
  L.max_tiles = (int)((P + bm - 1) / bm + (size_t)(E < (int)P ? E : (int)P));
  L.x_exp = 0;
  L.a_max = L.x_exp + moe_align_up((size_t)T * 4, 256);
  L.x16 = L.a_max + moe_align_up(P * 4, 256);
  L.a = L.x16 + moe_align_up((size_t)T * H * 2, 256);
  L.a16 = L.a + moe_align_up(P * (size_t)I * 2, 256);
  // 128-row down blocks read A converted to f16 (a copy beside A)
  L.total = L.a16 + (gate_up_msub(T, top_k, E, I) == 8 ? moe_align_up(P * (size_t)I * 2, 256) : 0);
  if (L.total < 256) L.total = 256;  // never empty, so T = 0 still gets a valid pointer
  return L;
}

// ---------------------------------------------------------------- prep ----
// One wave per token (prep_row, shared with the decode selection kernel); the
// other threads clear the per-row maximum of A.
template <bool NORM>
__global__ __launch_bounds__(kThreads) void k_prep(const uint16_t *__restrict__ x,
                                                   const uint16_t *__restrict__ norm_w, float eps,
                                                   int T, int H, int P, uint16_t *__restrict__ x16,
                                                   int32_t *__restrict__ x_exp,
                                                   uint32_t *__restrict__ a_max) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = blockIdx.x * kThreads + tid; i < P; i += gridDim.x * kThreads) a_max[i] = 0u;
  const int t = blockIdx.x * 4 + wave;
  if (t < T) prep_row<NORM>(x, norm_w, eps, H, t, x16, x_exp);
}

// gelu_tanh(g) = 0.5 g (1 + tanh(u)), u = sqrt(2/pi) (g + 0.044715 g^3), in the
// equal form g / (1 + exp(-2u)) (1 + tanh(u) = 2 / (1 + exp(-2u))): one
// hardware exp2 and one reciprocal (each about 1 ulp) instead of a tanh.
// Large |u| saturates correctly: exp -> inf gives 0, exp -> 0 gives g.
__device__ __forceinline__ float gelu_tanh(float g) {
  const float c2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float t = c2 * (g + 0.044715f * g * g * g);
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// acc += a * b on the matrix core with the accumulator kept in place in the
// accumulation registers (the "a" constraint), for kernels whose
// accumulators fill them.  The compiler still tracks the operands (it waits
// for the loads that produce a and b), but it does not know the statement is
// an MFMA, so the statement and its users carry the pipeline waits the
// compiler would otherwise insert:
//  * a VALU write of a, b or acc (the accumulators' zeroing included) needs
//    two wait states before an MFMA reads it: the s_nop 1 in front;
//  * an MFMA result read as the next MFMA's accumulator in the same
//    registers needs no wait (the compiler issues such chains back to back);
//  * an MFMA result read by anything else: mfma_acc_drain(), 24 wait states
//    (more than a 16x16x32 f16 MFMA needs) and a scheduling barrier, after
//    the last mfma_acc and before the accumulators are read.
__device__ __forceinline__ void mfma_acc(f32x4 &acc, const f16x8 &a, const f16x8 &b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The same without the two wait states, for an MFMA whose operands no VALU
// op has written in the two instructions before it (the caller pins that
// order with scheduling barriers).
__device__ __forceinline__ void mfma_acc_nw(f32x4 &acc, const f16x8 &a, const f16x8 &b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Zeroes the accumulators in the accumulation registers, then waits the two
// wait states after those writes, so that any MFMA may read them next.
template <int Q, int NW>
__device__ __forceinline__ void mfma_acc_zero(f32x4 (&acc)[Q][NW]) {
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      acc[q][i] = f32x4{0, 0, 0, 0};
      asm volatile("" : "+a"(acc[q][i]));
    }
  asm volatile("s_nop 1" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void mfma_acc_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------- grouped expert GEMM ----
// Tiled mode (prefill).  A workgroup (4 waves) owns one block of 16*MSUB
// sorted rows of one expert and 4*NP*16 output columns; each wave owns NP row
// tiles of 16 outputs (gated: NP gate tiles and the same NP up tiles).
//
// K advances in units of 128.  Per unit the activation block [rows][128] is
// staged once in LDS as f16 (gate/up: a ring of three buffers filled by
// direct buffer-to-LDS loads; down: double-buffered through registers) and
// shared by the 4 waves; each lane loads its 16 bytes of every weight row
// tile it owns (one contiguous kilobyte per wave in the tiled layout),
// dequantises them in registers and runs Q x NW x 4 MFMAs 16x16x32, so one
// LDS fragment feeds NW MFMAs and one dequantised weight fragment feeds Q.
// Q is the number of 16-row groups of the block that hold rows (a partial
// block at the end of an expert's bucket has fewer): the kernel picks the
// instantiation per workgroup, so empty groups are neither staged nor
// multiplied.  Gate/up waves whose columns lie past N stage activations for
// the others but issue no MFMAs.  Gate/up keeps the weights of two units and
// the activations of two units in flight while a unit is multiplied; down
// one unit of weights and two of activations.
//
// 128-row gate/up blocks (MSUB = 8) keep their 128 accumulators per wave in
// the accumulation registers through mfma_acc (below), the only way found to
// fit them beside the rest at two waves per SIMD: the compiler, left to
// itself, moved accumulators between register files or spilled them.
//
// Order of the workgroups: a 1-D grid, a multiple of the 8 XCDs.  Hardware
// hands workgroup b to XCD b % 8; each XCD walks one contiguous range of the
// logical order (expert, then groups of kRowGroup row blocks, and in a group
// column block, then row block), workgroup b taking block b / 8 of XCD
// b % 8's range.  Down cuts the order into ranges of equal block counts,
// gate/up into ranges of about equal cost (find_block).  The row blocks that reuse a column
// block's weights run side by side on one XCD and hit its L2 instead of HBM,
// and so do the column blocks that reuse a group's activations.
constexpr int kUnitK = 128;

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// Row blocks per group of the block order (below).
constexpr int kRowGroup = 8;

// 16-row groups multiplied for a block of `rows` rows (the kernel's
// dispatch below)
__device__ __forceinline__ int block_groups(int rows, int msub) {
  if (msub == 8) return rows > 64 ? 8 : rows > 32 ? 4 : rows > 16 ? 2 : 1;
  return rows > 48 ? 4 : rows > 32 ? 3 : rows > 16 ? 2 : 1;
}

// Cost of a block in the balanced split: kBlockCost + its 16-row groups (a
// block's weight stream, dequantisation and epilogue set-up do not depend on
// its rows).  Measured at 2048 tokens with Zipf routing, gate/up: 4 -> 185
// us, 6 -> 184, 8 -> 181 (equal-count ranges: 211).
constexpr int kBlockCost = 8;

// The block of this workgroup: expert e, row offset m0 in its bucket, column
// block cb; false when the workgroup has none.  Expert e holds
// ceil(M_e / bm) * ncb consecutive blocks of the block order (lane l takes
// experts PER*l .. PER*l + PER - 1; DPP prefix sums over the lanes, scalar
// results).  Workgroup b runs on XCD x = b % 8 as its j = b / 8-th
// workgroup and takes block j of XCD x's range of the order.
// BALANCED = false: 8 ranges of ceil(blocks / 8) blocks (the real block
// count: the grid is sized for the most blocks any routing can give, and
// ranges of gridDim.x / 8 left the last XCD with a few blocks or none).
// BALANCED = true: the ranges hold about equal cost (kBlockCost + 16-row
// groups per block), each at most gridDim.x / 8 blocks long; used where
// blocks with few rows are common beside full ones (the Zipf tail beside
// the head experts), whose count-equal ranges differ in work by up to a
// third.
template <bool BALANCED>
__device__ bool find_block(const int32_t *__restrict__ offsets, int E, int bm, int msub, int ncb,
                           int grp, int &e, int &m0, int &cb) {
  constexpr int PER = MOE_MAX_EXPERTS / kWave;  // 4
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(offsets, (uint32_t)(E + 1) * 4u);
  int off[PER + 1];
#pragma unroll
  for (int i = 0; i <= PER; ++i)
    off[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(ro, (uint32_t)(PER * lane + i) * 4u, 0, 0);
  int nblk[PER], sum = 0, cs[PER], csum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int n = PER * lane + i < E ? off[i + 1] - off[i] : 0;
    nblk[i] = (n + bm - 1) / bm;
    sum += nblk[i] * ncb;
    if (BALANCED) {
      const int full = n / bm, rem = n - full * bm;
      cs[i] = ncb * (full * (kBlockCost + msub) + (rem > 0 ? kBlockCost + block_groups(rem, msub) : 0));
      csum += cs[i];
    }
  }
  const int incl = wave_incl_scan(sum);
  const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
  const int excl = incl - sum;
  const int cap = (int)gridDim.x / kXcds, x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  int lo, hi;
  if (!BALANCED) {
    const int len = (total + kXcds - 1) / kXcds;
    lo = min(total, x * len);
    hi = min(total, lo + len);
  } else {
    // range starts s_1 .. s_7 at the blocks where the cost prefix reaches
    // y/8 of the total (uniform cost per block inside an expert), clamped so
    // that every range has at most cap blocks and the later XCDs can still
    // take the rest
    const int cincl = wave_incl_scan(csum);
    const int C = __builtin_amdgcn_readlane(cincl, kWave - 1), cexcl = cincl - csum;
    int prev = 0;
    lo = 0;
    hi = total;
    for (int y = 1; y < kXcds; ++y) {
      const int t = (int)((long long)y * C / kXcds);
      const unsigned long long bal = __ballot(t >= cexcl && t < cincl);
      int at = total;
      if (bal) {
        int cb0 = cexcl, bb0 = excl, r = -1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          if (r < 0 && t >= cb0 && t < cb0 + cs[i])
            r = bb0 + (int)((long long)(t - cb0) * (nblk[i] * ncb) / cs[i]);
          cb0 += cs[i];
          bb0 += nblk[i] * ncb;
        }
        at = __builtin_amdgcn_readlane(r, (int)__builtin_ctzll(bal));
      }
      const int sy = max(prev, max(min(at, prev + cap), total - (kXcds - y) * cap));
      if (y == x) lo = sy;
      if (y == x + 1) hi = sy;
      prev = sy;
    }
  }
  if (lo + j >= hi) return false;  // uniform
  const int L = lo + j;
  const int src = (int)__builtin_ctzll(__ballot(L >= excl && L < incl));
  int ee = 0, rem = 0, nb = 1, base = excl;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int n = nblk[i] * ncb;
    if (L >= base && L < base + n) {
      rem = L - base;
      ee = PER * lane + i;
      nb = nblk[i];
    }
    base += n;
  }
  e = __builtin_amdgcn_readlane(ee, src);
  rem = __builtin_amdgcn_readlane(rem, src);
  nb = __builtin_amdgcn_readlane(nb, src);
  // expert e's blocks in groups of grp row blocks (the last group may be
  // smaller), each group column-block major: gsz row blocks x ncb columns
  const int gi = rem / (grp * ncb);  // scalar
  const int gsz = min(grp, nb - gi * grp);
  const int r2 = rem - gi * grp * ncb;
  cb = r2 / gsz;
  m0 = (gi * grp + r2 - cb * gsz) * bm;
  return true;
}

// LDS layout of the activation block: [rows][128] f16, no padding; the
// 16-byte chunk c of row m sits at chunk position c ^ (m & 15), so the 16
// rows read by one MFMA fragment load (same c) hit 16 different bank groups.
__device__ __forceinline__ int lds_chunk(int m, int c) { return m * 16 + (c ^ (m & 15)); }

// Wait until at most n vector-memory loads of this wave are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their
// maxima, i.e. not waited for).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// Register budget of the K loop: weight register sets of the LDS-direct
// (gate/up) pipeline (3: weights two units ahead; 2: one unit ahead).  LDS
// activation buffers of that pipeline: kGemmLdsBufs - 1 units in flight.
constexpr int kGemmWeightSets = 3;
constexpr int kGemmLdsBufs = 3;
// 128-row blocks (MSUB = 8, for buckets of many rows): each wave keeps 8 row
// groups x 4 weight row tiles (gate/up: 2 gate + 2 up; down: 4) = 128
// accumulators, which fill the accumulation registers (mfma_acc), so each
// dequantised weight fragment feeds 8 MFMAs instead of 4 -- half the dequant
// VALU work per MFMA.  The other 128 registers of a wave at two waves per
// SIMD then hold one activation fragment set and two weight sets; the
// activations come through a two-buffer LDS ring (64 KB: two workgroups per
// CU) filled by direct loads, for down from a copy of A converted to f16.
template <int MSUB>
constexpr int gemm_weight_sets() { return MSUB == 8 ? 2 : kGemmWeightSets; }

// LDS activation buffers of the tiled-mode kernels
template <int MSUB, bool GATED>
constexpr int gemm_lds_bufs() { return MSUB == 8 ? 2 : GATED ? kGemmLdsBufs : 2; }

// One block of the tiled mode: rows row0 .. row0 + mrows - 1 (mrows <= 16 Q)
// of expert e, column block cb.  Q: the 16-row groups holding rows; only
// those are staged, multiplied and stored.  s_a: the LDS activation buffers
// [gemm_lds_bufs][16 MSUB * kUnitK]; s_rowscale: [16 MSUB].
// DIRECT: the activations are f16 in memory (gate/up; down with 128-row
// blocks, whose A was converted to f16 beforehand): buffer loads write
// them straight into LDS (no registers).  Otherwise (down, bf16 A): they go
// through registers and are converted to f16 with the row's power of two.
template <int MSUB, int Q, int NP, bool GATED, int FMT>
__device__ __forceinline__ void gemm_run(
    const uint16_t *__restrict__ a_src, const int32_t *__restrict__ x_exp,
    uint32_t *__restrict__ a_max, const int32_t *__restrict__ sorted_pairs, int top_k,
    uint32_t a_bytes, const Nvfp4 &w0, const Nvfp4 &w1, int K, int N, uint16_t *__restrict__ out,
    int e, int row0, int mrows, int cb, uint16_t (*s_a)[kBM * MSUB * kUnitK], float *s_rowscale) {
  constexpr bool DIRECT = GATED || MSUB == 8;
  constexpr int BM = kBM * MSUB;
  constexpr int NW = GATED ? 2 * NP : NP;  // weight row tiles streamed by a wave
  using WF = WeightFmt<FMT>;
  constexpr int SB = WF::kScaleBytes;       // scale bytes per lane and K unit
  constexpr int NBUF = gemm_lds_bufs<MSUB, GATED>();  // LDS activation buffers
  // wave: uniform (a scalar register), so the LDS destinations of the
  // staging loads are computed on the scalar unit
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int nunits = (K + kUnitK - 1) / kUnitK;
  const int nt0 = (cb * 4 + wave) * NP;          // first output row tile of this wave
  const bool wave_on = nt0 * 16 < N;  // waves past the last column stage only (gate/up: no MFMAs)

  // ---- weight streams of this wave (buffer resources over expert e's
  // tensors; lanes past K, units past the end and waves past N read zeros)
  __amdgpu_buffer_rsrc_t rw[NW], rs[NW];
  uint32_t vw[NW], vs[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const Nvfp4 &w = (GATED && i >= NP) ? w1 : w0;
    const int nt = nt0 + (GATED ? i % NP : i);
    rw[i] = make_rsrc(w.packed + (size_t)e * N * (K / 2), (uint32_t)((size_t)N * (K / 2)));
    rs[i] = make_rsrc(w.scales + (size_t)e * N * K * SB / 32, (uint32_t)((size_t)N * K * SB / 32));
    vw[i] = wave_on ? (uint32_t)nt * 16 * (K / 2) + lane * 16 : kOOB;
    vs[i] = wave_on ? (uint32_t)nt * K * SB / 2 + lane * SB : kOOB;
  }
  auto load_w = [&](int u, u32x4 (&wv)[NW], uint32_t (&sv)[NW]) {
    const bool ok = u < nunits && u * kUnitK + 32 * g < K;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      // a plain load: the row blocks of a block group reuse these weights
      // from L2 (streamed loads measured 7% slower at 16384 tokens)
      wv[i] = bload16(rw[i], off_if(ok, vw[i] + (uint32_t)u * 1024));
      sv[i] = load_scale<SB>(rs[i], off_if(ok, vs[i] + (uint32_t)u * 64 * SB));
    }
  };

  // weight register sets; unit 0's weights are requested first, before the
  // staging map looks up the block's rows (they do not depend on them)
  constexpr int WS = DIRECT ? gemm_weight_sets<MSUB>() : 2;
  u32x4 wv[WS][NW];
  uint32_t sv[WS][NW];
  load_w(0, wv[0], sv[0]);
  __builtin_amdgcn_sched_barrier(0);

  // ---- staging map.  DIRECT: load q of wave w fills rows 16q + 4w + lane/16,
  // LDS chunk positions lane%16 (one contiguous kilobyte per load); the lane
  // fetches the K chunk that belongs at that position.  Otherwise: thread ->
  // (row 16q + tid/16, K chunk tid%16).  Rows past the block, and chunks past
  // K, read hardware zeros (offset out of range).
  const int st_row = DIRECT ? 4 * wave + (lane >> 4) : (tid >> 4);  // row within each 16
  const int st_c = DIRECT ? ((lane & 15) ^ st_row) : (tid & 15);      // K chunk of this lane
  uint32_t st_off[Q];
  float st_scale[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int m = q * kBM + st_row;
    const bool ok = m < mrows;
    const int prow = ok ? row0 + m : row0;
    const int arow = GATED ? sorted_pairs[prow] / top_k : prow;
    st_off[q] = ok ? (uint32_t)arow * (uint32_t)K * 2 + (uint32_t)st_c * 16 : kOOB;
    st_scale[q] = 1.0f;
    if (!GATED) st_scale[q] = __builtin_ldexpf(1.0f, 14 - row_exponent(__uint_as_float(a_max[prow])));
  }
  // per-row factor applied to the fp32 sums: 2^(exponent - 14)
  if (tid < BM) {
    float f = 0.0f;
    if (tid < mrows) {
      const int ex = GATED ? x_exp[sorted_pairs[row0 + tid] / top_k]
                           : row_exponent(__uint_as_float(a_max[row0 + tid]));
      f = __builtin_ldexpf(1.0f, ex - 14);
    }
    s_rowscale[tid] = f;
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_src, a_bytes);
  auto a_offset = [&](int u, int q) -> uint32_t {
    const bool kok = u < nunits && u * kUnitK + st_c * 8 < K;
    return off_if(kok, st_off[q] + (uint32_t)u * kUnitK * 2);  // kOOB + 256u stays out of range
  };
  // DIRECT staging of unit u into buffer b
  auto load_a_lds = [&](int u, int b) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void *)&s_a[b][(q * kBM + 4 * wave) * kUnitK], 16,
          a_offset(u, q), 0, 0, 0);
  };
  // register staging
  auto load_a = [&](int u, u32x4 (&v)[Q]) {
#pragma unroll
    for (int q = 0; q < Q; ++q) v[q] = bload16(ra, a_offset(u, q));
  };
  auto store_a = [&](int b, const u32x4 (&v)[Q]) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      u32x4 o = v[q];
      if (!GATED) {  // bf16 -> f16 with the row's power of two (exact)
        const float f = st_scale[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f16 lo = (f16)(__uint_as_float(v[q][i] << 16) * f);
          const f16 hi = (f16)(__uint_as_float(v[q][i] & 0xFFFF0000u) * f);
          o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
      }
      *(u32x4 *)(&s_a[b][lds_chunk(q * kBM + st_row, st_c) * 8]) = o;
    }
  };

  f32x4 acc[Q][NW];
  if constexpr (MSUB == 8) {
    mfma_acc_zero(acc);
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < NW; ++i) acc[q][i] = f32x4{0, 0, 0, 0};
  }

  // One K unit: 4 steps of 32.  The weights of step j + 1 are dequantised
  // while the MFMAs of step j run (two register sets), and scheduling-group
  // barriers interleave one MFMA with two VALU ops so that the VALU and the
  // matrix core work side by side.  The activation fragment q of step j is
  // row 16q + r, K chunk 4g + j: lds_chunk(16q + r, c) = lds_chunk(r, c) +
  // 256 q, so one address per step serves every q (immediate offsets).
  auto compute = [&](const uint16_t *abuf, const u32x4 (&wv)[NW], const uint32_t (&sv)[NW]) {
    typename WF::Prep bs[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) bs[i] = WF::prep(sv[i]);
    if constexpr (MSUB == 8) {
      // 128-row blocks (accumulators in the accumulation registers, updated
      // in place by mfma_acc).  One activation fragment set: fragment q of
      // step j + 1 is read from LDS right after its last MFMA of step j.
      // Weight tile s + 1 (step-major order) is dequantised while the Q MFMAs
      // of tile s run; for NVFP4 its 8 VALU ops are placed one after each
      // MFMA (scheduling barriers keep that order).
      f16x8 a[Q], b[2];
#pragma unroll
      for (int q = 0; q < Q; ++q)
        a[q] = __builtin_bit_cast(f16x8, *(const u32x4 *)(abuf + lds_chunk(r, 4 * g) * 8 + q * kBM * kUnitK));
      b[0] = WF::dequant(wv[0][0], bs[0], 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          const int st = j * NW + i;
          const bool next = st + 1 < 4 * NW;
          const int ni = (i + 1) % NW, nj = j + (i + 1) / NW;
          constexpr bool kSpread = FMT == MOE_FORMAT_NVFP4;
          if (!kSpread && next) b[(st + 1) & 1] = WF::dequant(wv[ni][nj], bs[ni], nj);
          f16x2 c[4];
          const uint32_t wn = wv[ni][nj];
          f16x2 ss = {};
          if constexpr (kSpread) ss = f16x2{bs[ni].s[nj >> 1], bs[ni].s[nj >> 1]};
          auto deq_step = [&](int k) {  // k: a constant once the loops are unrolled
            switch (k) {
              case 0: c[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wn, 1.0f, 0); break;
              case 2: c[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wn, 1.0f, 1); break;
              case 4: c[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wn, 1.0f, 2); break;
              case 6: c[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wn, 1.0f, 3); break;
              default: c[k >> 1] = c[k >> 1] * ss;
            }
          };
#pragma unroll
          for (int q = 0; q < Q; ++q) {
            // the tile's first MFMA reads b just completed by a VALU op; the
            // later ones follow a dequant step writing the next tile's
            // registers, or an LDS read (waited for by counter)
            if (kSpread && q > 0) mfma_acc_nw(acc[q][i], a[q], b[st & 1]);
            else mfma_acc(acc[q][i], a[q], b[st & 1]);
            if (i == NW - 1 && j < 3)
              a[q] = __builtin_bit_cast(
                  f16x8, *(const u32x4 *)(abuf + lds_chunk(r, 4 * g + j + 1) * 8 + q * kBM * kUnitK));
            if (kSpread && next && q < 8) deq_step(q);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (kSpread && next) {
#pragma unroll
            for (int k = Q; k < 8; ++k) deq_step(k);
            b[(st + 1) & 1] = f16x8{c[0][0], c[0][1], c[1][0], c[1][1], c[2][0], c[2][1], c[3][0], c[3][1]};
          }
        }
      }
      return;
    }
    f16x8 a[Q], b[2][NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) b[0][i] = WF::dequant(wv[i][0], bs[i], 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t *aj = abuf + lds_chunk(r, 4 * g + j) * 8;
#pragma unroll
      for (int q = 0; q < Q; ++q)
        a[q] = __builtin_bit_cast(f16x8, *(const u32x4 *)(aj + q * kBM * kUnitK));
      if (j < 3) {
#pragma unroll
        for (int i = 0; i < NW; ++i) b[(j + 1) & 1][i] = WF::dequant(wv[i][j + 1], bs[i], j + 1);
      }
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int i = 0; i < NW; ++i) acc[q][i] = mfma16x16x32(a[q], b[j & 1][i], acc[q][i]);
      __builtin_amdgcn_sched_group_barrier(0x100, Q, 0);
      if (j < 3) {
#pragma unroll
        for (int m = 0; m < Q * NW; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (8 * NW) / (Q * NW), 0);
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, Q * NW, 0);
      }
    }
  };

  // ---- pipeline, one barrier per unit; unrolled so that register buffers
  // have static indices (steps past the last unit multiply nothing or
  // zeros).  DIRECT (gate/up): below.  Otherwise (down): weights
  // double-buffered in registers, unit u+1 issued before unit u is
  // multiplied; activations in two register sets, unit u+3 loaded when unit
  // u+1 has been converted into the LDS double buffer.
  if (DIRECT) {
    // activations NBUF - 1 units ahead (a ring of NBUF LDS buffers), weights
    // WS - 1 units ahead (WS register sets); the loop is unrolled by a
    // multiple of NBUF and of WS, and the steps past the last unit skip
    // their MFMAs (a uniform branch).  Every iteration issues Q
    // activation loads, then 2 NW weight and scale loads, all unconditional
    // (past the end they read zeros), so the vector-memory counter waits
    // below are exact: after the activations of a unit come the NBUF - 2
    // later units' activation loads and, before it is needed, at least
    // min(NBUF - 1, WS) groups of weight loads.  (Unit 0's weights went
    // first, before the activation loads of units 0 .. NBUF - 2; then units
    // 1 .. WS - 2 of the weights.)
    static_assert(WS >= 2, "");
    constexpr int UNR = NBUF * WS / gcd_c(NBUF, WS);
    constexpr int PRE = (NBUF - 2) * Q + (WS - 2) * 2 * NW;  // after unit 0's activations
    constexpr int AHEAD = (NBUF - 2) * Q + (NBUF - 1 < WS ? NBUF - 1 : WS) * 2 * NW;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) load_a_lds(i, i);
#pragma unroll
    for (int i = 1; i < WS - 1; ++i) load_w(i, wv[i], sv[i]);
    MOE_WAIT_VMCNT(PRE);  // unit 0 of the activations (and of the weights) has landed
    __syncthreads();
    // Units past the last one (up to UNR - 1 of them) multiply zeros; waves
    // past N run a copy of the loop without MFMAs (no branch inside the loop)
    const int nuu = (nunits + UNR - 1) / UNR * UNR;
    auto k_loop = [&](auto on) {
      for (int u0 = 0; u0 < nuu; u0 += UNR) {
#pragma unroll
        for (int d = 0; d < UNR; ++d) {
          const int u = u0 + d;  // LDS ring buffer of unit u: u % NBUF = d % NBUF
          load_a_lds(u + NBUF - 1, (d + NBUF - 1) % NBUF);
          load_w(u + WS - 1, wv[(d + WS - 1) % WS], sv[(d + WS - 1) % WS]);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (decltype(on)::value) compute(s_a[d % NBUF], wv[d % WS], sv[d % WS]);
          __builtin_amdgcn_sched_barrier(0);
          MOE_WAIT_VMCNT(AHEAD);  // unit u+1 of the activations has landed
          __syncthreads();
        }
      }
    };
    if (wave_on) k_loop(std::true_type{});
    else k_loop(std::false_type{});
  } else {
    const int nu = (nunits + 1) & ~1;
    u32x4 av[2][Q];
    load_a(0, av[0]);  // unit 0's weights are already in flight
    load_a(1, av[1]);
    store_a(0, av[0]);
    load_a(2, av[0]);
    __syncthreads();
    for (int u0 = 0; u0 < nu; u0 += 2) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int u = u0 + d;
        load_w(u + 1, wv[d ^ 1], sv[d ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        compute(s_a[d], wv[d], sv[d]);  // no branch: it would split the pipelined loop
        __builtin_amdgcn_sched_barrier(0);
        store_a(d ^ 1, av[d ^ 1]);
        load_a(u + 3, av[d ^ 1]);
        __syncthreads();
      }
    }
  }
  if (!wave_on) return;  // no barrier follows
  if constexpr (MSUB == 8) mfma_acc_drain();

  // ---- epilogue: lane holds rows 16q + 4g + jj, column r of each row tile.
  // The block's output rows go through a buffer resource: rows past the
  // block and columns past N get offsets outside it (the hardware drops those
  // stores), so no store sits under a branch and each takes one 32-bit
  // offset (a row's, plus its column's).
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + (size_t)row0 * N, (uint32_t)((size_t)mrows * N * 2));
  uint32_t coff[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int n = (nt0 + i) * 16 + r;
    coff[i] = n < N ? (uint32_t)n * 2 : 0x40000000u;  // plus a row offset or kOOB: no wrap
  }
  if (GATED) {
    const float gg = FMT == MOE_FORMAT_NVFP4 ? w0.global[e] : 1.0f;
    const float gu = FMT == MOE_FORMAT_NVFP4 ? w1.global[e] : 1.0f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = q * kBM + 4 * g + jj;
        const bool ok = m < mrows;
        const float f = s_rowscale[m];
        const uint32_t roff = ok ? (uint32_t)(m * N) * 2 : kOOB;
        uint32_t rmax = 0;  // max |A| of the row (f32 bits)
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const float G = acc[q][i][jj] * (gg * f), U = acc[q][NP + i][jj] * (gu * f);
          const uint16_t ab = f32_to_bf16_rne(gelu_tanh(G) * U);
          __builtin_amdgcn_raw_buffer_store_b16(ab, ro, roff + coff[i], 0, 0);
          rmax = max(rmax, ok ? bf16_abs_bits(ab) : 0u);
        }
        // the row maxima of A: 128-row blocks leave them to k_a_f16, which
        // reads every row of A anyway
        if constexpr (MSUB != 8) {
          rmax = row16_max_u32(rmax);
          if (r == 0 && ok) atomicMax(&a_max[row0 + m], rmax);
        }
      }
    }
  } else {
    const float gd = FMT == MOE_FORMAT_NVFP4 ? w0.global[e] : 1.0f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = q * kBM + 4 * g + jj;
        const float f = gd * s_rowscale[m];  // 0 past the block's rows
        const uint32_t roff = m < mrows ? (uint32_t)(m * N) * 2 : kOOB;
#pragma unroll
        for (int i = 0; i < NP; ++i)
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(acc[q][i][jj] * f), ro, roff + coff[i], 0, 0);
      }
    }
  }
}

template <int MSUB, int NP, bool GATED, int FMT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_expert_gemm(
    const uint16_t *__restrict__ a_src,  // GATED: x16 [T][K] f16; else A [P][K] bf16
    const int32_t *__restrict__ x_exp,   // GATED: exponent of each token
    uint32_t *__restrict__ a_max,        // GATED: row max of A (written); else read
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ sorted_pairs, int top_k,
    int E, int ncb, uint32_t a_bytes,
    Nvfp4 w0, Nvfp4 w1,                  // GATED: gate, up; else w0 = down
    int K, int N, uint16_t *__restrict__ out) {
  static_assert(MSUB == 4 || MSUB == 8, "one instantiation per 16-row group count below");
  constexpr int BM = kBM * MSUB;
  __shared__ __attribute__((aligned(16))) uint16_t s_a[gemm_lds_bufs<MSUB, GATED>()][BM * kUnitK];
  __shared__ float s_rowscale[BM];
  int e, m0, cb;
  // gate/up: cost-balanced XCD ranges; down (short blocks, whose start-up
  // latency the balanced split's extra work would add to): equal counts
  if (!find_block<GATED>(offsets, E, BM, MSUB, ncb, kRowGroup, e, m0, cb)) return;  // uniform
  const int row0 = offsets[e] + m0;
  const int mrows = min(BM, offsets[e + 1] - row0);  // >= 1: a block holds rows
#define MOE_GEMM_RUN(Q)                                                                          \
  gemm_run<MSUB, Q, NP, GATED, FMT>(a_src, x_exp, a_max, sorted_pairs, top_k, a_bytes, w0, w1, K, \
                                    N, out, e, row0, mrows, cb, s_a, s_rowscale)
  // the 16-row groups holding rows (uniform)
  if constexpr (MSUB == 4) {
    if (mrows > 3 * kBM) MOE_GEMM_RUN(4);
    else if (mrows > 2 * kBM) MOE_GEMM_RUN(3);
    else if (mrows > kBM) MOE_GEMM_RUN(2);
    else MOE_GEMM_RUN(1);
  } else {
    if (mrows > 4 * kBM) MOE_GEMM_RUN(8);
    else if (mrows > 2 * kBM) MOE_GEMM_RUN(4);
    else if (mrows > kBM) MOE_GEMM_RUN(2);
    else MOE_GEMM_RUN(1);
  }
#undef MOE_GEMM_RUN
}

// For the 128-row down blocks: the row maxima of A (a_max, which the 128-row
// gate/up blocks do not compute) and A [P][I] bf16 -> f16 times its row's
// power of two 2^(14 - exponent of max|A|) (exact, as the 64-row kernel
// converts it while staging), once per element instead of once per column
// block, so that the down kernel stages A into LDS with direct loads.  One
// half-wave per row, which it holds in registers (NCH 16-byte chunks per
// lane): the row's maximum, then its conversion.
template <int NCH>
__global__ __launch_bounds__(kThreads) void k_a_f16(const uint16_t *__restrict__ a,
                                                    uint32_t *__restrict__ a_max, int P,
                                                    int I, uint16_t *__restrict__ a16) {
  constexpr int L = kWave / 2;  // lanes per row
  const int lane = threadIdx.x & (L - 1);
  const int per_row = I / 8;  // 16-byte chunks per row, at most L NCH
  const int row = blockIdx.x * (kThreads / L) + (int)(threadIdx.x / L);
  const bool on = row < P;  // both halves of a wave stay for the shuffles
  const uint16_t *ar = a + (size_t)(on ? row : 0) * I;
  u32x4 v[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + k * L;
    v[k] = (on && c < per_row) ? *(const u32x4 *)(ar + c * 8) : u32x4{0, 0, 0, 0};
  }
  uint32_t mx = 0;  // max |A| of the row (f32 bits; NaN counts as 0)
#pragma unroll
  for (int k = 0; k < NCH; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mx = max(mx, max(bf16_abs_bits((uint16_t)v[k][i]), bf16_abs_bits((uint16_t)(v[k][i] >> 16))));
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
  if (!on) return;
  if (lane == 0) a_max[row] = mx;
  const float f = __builtin_ldexpf(1.0f, 14 - row_exponent(__uint_as_float(mx)));
  {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = lane + k * L;
      if (c >= per_row) break;
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16 lo = (f16)(__uint_as_float(v[k][i] << 16) * f);
        const f16 hi = (f16)(__uint_as_float(v[k][i] & 0xFFFF0000u) * f);
        o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *(u32x4 *)(a16 + (size_t)row * I + c * 8) = o;
    }
  }
}

// ------------------------------------------------------- GEMV mode ----
// Few rows per expert (decode).  A workgroup owns NW weight row tiles (gated:
// NP gate tiles and the same NP up tiles; down: NP tiles) of one tile of up
// to ROWS sorted rows of one expert; its 4 waves split K (a quarter of the K
// units each), stream their share with no LDS staging and no barrier, and
// add their partial sums in LDS once at the end (in wave order).  Short
// per-wave streams and many waves keep HBM busy even when a decode batch
// touches few experts.
//
// Packing of R = 4, 8 or 16 rows into one 16x16x32 MFMA output block: the
// 16 accumulator rows are 16/R groups of R rows.  Lane (r, g) serves row
// r % R of group h = r / R and loads NL = R/4 adjacent 16-byte chunks of it,
// K = 128u + 32g + 8(h NL + s), s < NL; it feeds chunk s to MFMA
// j = h NL + s and zeros to the others.  MFMA j multiplies by dword j of the
// lane's weight bytes (K = 128u + 32g + 8j), so group h accumulates the K
// chunks j in [h NL, h NL + NL) of its rows; the groups are summed once after
// the K loop.  Every tile costs 4 MFMAs per weight row tile and K unit, and
// R/4 activation loads per lane.  Units up to kGemvPD ahead are in flight.
//
// Weight row tiles per wave (NP): every tile of a wave shares the wave's
// activation loads, and each activation load costs the CU about as much as a
// weight load, so more tiles per wave pay off where a unit needs several
// activation loads (16-row tiles) or where the K split is on.  Gate/up (K =
// hidden, long) always takes the K split with 2 gate + 2 up tiles per wave:
// 4x the waves of the unsplit layout, each with a quarter of K.  Down (K =
// expert intermediate, short) keeps whole-K waves unless its grid is small.
constexpr int kGemvPD = 1;
constexpr int kGateNP = 2;       // gate/up row-tile pairs per wave (K split)
constexpr int kDownNP = 2;       // down row tiles per wave (8-row tiles)
constexpr int kDownNPMany = 4;   // ... when there are many tiles (P >= 3E)
constexpr int kDownNPWide = 4;   // ... with 16-row tiles
// down takes the K split when the unsplit grid would have fewer workgroups
// (T = 1: 198 workgroups unsplit, the split slightly faster; T = 4: 792, the
// unsplit grid faster)
constexpr int kGemvSplitBelow = 512;


template <int NL, int NW>
struct GemvUnit {
  u32x4 a[NL];
  u32x4 w[NW];
  uint32_t s[NW];
};

struct GemvArgs {
  const uint16_t *a_src;   // GATED: x16 [T][K] f16; else A [P][K] bf16
  const int32_t *x_exp;    // GATED: exponent of each token
  uint32_t *a_max;         // GATED: written; else read
  const int32_t *sorted_pairs;
  int top_k, K, N, P;
  uint32_t a_bytes;        // bytes of a_src
  uint16_t *out;           // GATED: A [P][N] bf16; else Y [P][N] bf16
};

// STORE = false (down, one row: mrows == 1): instead of writing Y, lanes
// 0..15 return the row's bf16 outputs (as floats) of columns (nt0 + i) * 16 +
// lane in yout[i]; the other lanes' yout is undefined.
template <int R, int NP, bool GATED, int KS, int FMT, int PD = kGemvPD, bool STORE = true>
__device__ __forceinline__ void gemv_run(const GemvArgs &p, const Nvfp4 &w0, const Nvfp4 &w1,
                                         int e, int row0, int mrows, int nt0, float *s_red,
                                         float *yout = nullptr) {
  constexpr int NW = GATED ? 2 * NP : NP;
  constexpr int NL = R / 4;  // activation chunks per lane and unit
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4, h = r / R, m = r % R;
  const int K = p.K, N = p.N;
  const int nunits = (K + kUnitK - 1) / kUnitK;
  // this wave's share of the K units (KS = 4: the waves split K and their
  // partial sums meet in LDS after the loop; KS = 1: all of K)
  const int ub = KS == 1 ? 0 : wave * nunits / KS, ue = KS == 1 ? nunits : (wave + 1) * nunits / KS;

  using WF = WeightFmt<FMT>;
  constexpr int SB = WF::kScaleBytes;  // scale bytes per lane and K unit
  const float ep_g0 = FMT == MOE_FORMAT_NVFP4 ? w0.global[e] : 1.0f;
  const float ep_g1 = !GATED ? 0.0f : FMT == MOE_FORMAT_NVFP4 ? w1.global[e] : 1.0f;

  // weight streams: expert e's tensors through buffer resources; offsets past
  // the end (lanes past K, units past the end) read hardware zeros
  __amdgpu_buffer_rsrc_t rw[NW], rs[NW];
  uint32_t vw[NW], vs[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const Nvfp4 &w = (GATED && i >= NP) ? w1 : w0;
    const int nt = nt0 + (GATED ? i % NP : i);
    rw[i] = make_rsrc(w.packed + (size_t)e * N * (K / 2), (uint32_t)((size_t)N * (K / 2)));
    rs[i] = make_rsrc(w.scales + (size_t)e * N * K * SB / 32, (uint32_t)((size_t)N * K * SB / 32));
    vw[i] = (uint32_t)nt * 16 * (K / 2) + lane * 16;
    vs[i] = (uint32_t)nt * K * SB / 2 + lane * SB;
  }
  auto load_w = [&](int u, GemvUnit<NL, NW> &d) {
    const bool kok = u < ue && u * kUnitK + 32 * g < K;
    const uint32_t ow = kok ? (uint32_t)u * 1024 : kOOB, os = kok ? (uint32_t)u * 64 * SB : kOOB;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      d.w[i] = bload16_nt(rw[i], vw[i] + ow);
      d.s[i] = load_scale<SB>(rs[i], vs[i] + os);
    }
  };

  // ---- K-loop buffers; the first units' weight loads leave before this
  // lane's activation row is looked up (they do not depend on it), so their
  // latency overlaps that lookup
  constexpr int NB = PD + 1;
  GemvUnit<NL, NW> buf[NB];
#pragma unroll
  for (int d = 0; d < PD; ++d) load_w(ub + d, buf[d]);
  __builtin_amdgcn_sched_barrier(0);

  // activation row of this lane
  const bool row_ok = m < mrows;
  const int prow = row_ok ? row0 + m : row0;
  const int arow = GATED ? p.sorted_pairs[prow] / p.top_k : prow;
  const uint32_t va = row_ok ? (uint32_t)arow * (uint32_t)K * 2 + (uint32_t)(32 * g + 8 * h * NL) * 2
                             : kOOB;
  // the power of two of this lane's activation row: GATED, the token's
  // exponent (the row was rescaled by prep); else from the row's max |A|.
  // Requested here, used after the K loop: the epilogue takes the exponent of
  // its row 4g + jj from lane 4g + jj (whose activation row it is).
  int row_ex = 0;
  float a_scale = 1.0f;
  if (GATED) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x_exp, (uint32_t)(p.P / p.top_k) * 4u);
    row_ex = (int)__builtin_amdgcn_raw_buffer_load_b32(rx, row_ok ? (uint32_t)arow * 4u : kOOB, 0, 0);
  } else {
    row_ex = row_exponent(__uint_as_float(p.a_max[prow]));
    a_scale = __builtin_ldexpf(1.0f, 14 - row_ex);
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a_src, p.a_bytes);
  auto load_a = [&](int u, GemvUnit<NL, NW> &d) {
    const bool kok = u < ue && u * kUnitK + 32 * g < K;
    // va is kOOB for rows past the tile; kOOB + 256u + 16s stays out of range
    const uint32_t oa = kok ? va + (uint32_t)u * kUnitK * 2 : kOOB;
#pragma unroll
    for (int sl = 0; sl < NL; ++sl) d.a[sl] = bload16(ra, oa + 16 * sl);
  };
  auto load = [&](int u, GemvUnit<NL, NW> &d) {
    load_a(u, d);
    load_w(u, d);
  };
  f32x4 acc[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) acc[i] = f32x4{0, 0, 0, 0};
  auto compute = [&](const GemvUnit<NL, NW> &c) {
    f16x8 a[NL];
#pragma unroll
    for (int sl = 0; sl < NL; ++sl) {
      if (GATED) {
        a[sl] = __builtin_bit_cast(f16x8, c.a[sl]);
      } else {  // bf16 -> f16 with the row's power of two (exact)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          a[sl][2 * t] = (f16)(__uint_as_float(c.a[sl][t] << 16) * a_scale);
          a[sl][2 * t + 1] = (f16)(__uint_as_float(c.a[sl][t] & 0xFFFF0000u) * a_scale);
        }
      }
    }
    typename WF::Prep bs[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) bs[i] = WF::prep(c.s[i]);
    const f16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // this lane's operand for MFMA j: its chunk j - h NL when that is in range
      const f16x8 aj = NL == 4 ? a[j % NL] : (j / NL == h ? a[j % NL] : zero);
#pragma unroll
      for (int i = 0; i < NW; ++i) acc[i] = mfma16x16x32(aj, WF::dequant(c.w[i][j], bs[i], j), acc[i]);
    }
  };

  // ---- K loop: PD + 1 register buffers.  The loads of unit u + PD are
  // issued before unit u is multiplied (a scheduling barrier keeps them
  // there), so PD units stay in flight while a wave computes.  The unit
  // count is rounded up to a multiple of the buffer count; the extra units
  // read zeros through the buffer range check and add nothing.
#pragma unroll
  for (int d = 0; d < PD; ++d) load_a(ub + d, buf[d]);
  const int nu = (ue - ub + NB - 1) / NB * NB;
  for (int u0 = ub; u0 < ub + nu; u0 += NB) {
#pragma unroll
    for (int d = 0; d < NB; ++d) {
      load(u0 + d + PD, buf[(d + PD) % NB]);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- the K split: partial sums to LDS, wave 0 adds them in wave order
  // (a fixed order: the result is the same on every run) and finishes
  if (KS > 1) {
#pragma unroll
    for (int i = 0; i < NW; ++i)
      *(f32x4 *)&s_red[((wave * 64 + lane) * NW + i) * 4] = acc[i];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < KS; ++w)
#pragma unroll
      for (int i = 0; i < NW; ++i) acc[i] += *(const f32x4 *)&s_red[((w * 64 + lane) * NW + i) * 4];
  }

  // ---- sum the row groups: lane (n, g) holds accumulator rows 4g + jj =
  // group (4g + jj) / R, row (4g + jj) % R; after the butterfly over the
  // groups, lanes with 4g + jj < R hold the full sums of row 4g + jj.
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float t = acc[i][jj];
      if (R <= 8) t += __shfl_xor(t, 32, kWave);
      if (R <= 4) t += __shfl_xor(t, 16, kWave);
      acc[i][jj] = t;
    }

  // exponent of the epilogue rows 4g + jj (lane 4g + jj holds row 4g + jj)
  int ep_ex[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) ep_ex[jj] = __shfl(row_ex, (4 * g + jj) & 15, kWave);

  if (GATED) {
    const float gg = ep_g0, gu = ep_g1;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int mr = 4 * g + jj;  // row of this lane's sums (valid when mr < R)
      const bool ok = mr < R && mr < mrows;
      const float f = ok ? __builtin_ldexpf(1.0f, ep_ex[jj] - 14) : 0.0f;
      uint32_t rmax = 0;  // max |A| of the row (f32 bits)
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const float G = acc[i][jj] * (gg * f), U = acc[NP + i][jj] * (gu * f);
        const uint16_t ab = f32_to_bf16_rne(gelu_tanh(G) * U);
        // columns past N: a last column group of 3 row-tile pairs when N % 48 != 0
        const bool cok = ok && (nt0 + i) * 16 < N;
        if (cok) p.out[(size_t)(row0 + mr) * N + (nt0 + i) * 16 + r] = ab;
        rmax = max(rmax, cok ? bf16_abs_bits(ab) : 0u);
      }
      rmax = row16_max_u32(rmax);
      if (r == 0 && ok) atomicMax(&p.a_max[row0 + mr], rmax);
    }
  } else if (!STORE) {
    const float f = ep_g0 * __builtin_ldexpf(1.0f, ep_ex[0] - 14);  // row 0: lanes 0..15, jj = 0
#pragma unroll
    for (int i = 0; i < NP; ++i) yout[i] = __uint_as_float((uint32_t)f32_to_bf16_rne(acc[i][0] * f) << 16);
  } else {
    const float gd = ep_g0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int mr = 4 * g + jj;
      if (mr < R && mr < mrows) {
        const float f = gd * __builtin_ldexpf(1.0f, ep_ex[jj] - 14);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int n = (nt0 + i) * 16 + r;
          if (n < N) p.out[(size_t)(row0 + mr) * N + n] = f32_to_bf16_rne(acc[i][jj] * f);
        }
      }
    }
  }
}

// Tile y of the GEMV grid, for "expert e contributes ceil(M_e / rows) tiles
// of rows rows, in expert order": each wave finds it from the expert offsets
// (E + 1 ints) with a DPP prefix sum over the per-expert tile counts --
// about the latency of one load, so no separate tile-list kernel.  Lane l
// takes experts PER*l .. PER*l + PER - 1 and holds off[i] = offsets[PER*l + i]
// (any value past E).  Returns false when y is at or past the tile count
// (uniform).
constexpr int kTilePer = MOE_MAX_EXPERTS / kWave;  // 4
__device__ __forceinline__ bool find_tile_from(const int (&off)[kTilePer + 1], int E, int rows,
                                               int y, int &e, int &row0, int &mrows) {
  constexpr int PER = kTilePer;
  const int lane = threadIdx.x & 63;
  int c[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = PER * lane + i < E ? (off[i + 1] - off[i] + rows - 1) / rows : 0;
    sum += c[i];
  }
  const int incl = wave_incl_scan(sum);
  const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
  if (y >= total) return false;
  const int excl = incl - sum;
  const unsigned long long hit = __ballot(y >= excl && y < incl);
  const int src = (int)__builtin_ctzll(hit);
  // the owning lane resolves which of its experts and which tile of it
  int ee = 0, r0 = 0, mr = 0, base = excl;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (y >= base && y < base + c[i]) {
      const int t = y - base;
      ee = PER * lane + i;
      r0 = off[i] + t * rows;
      mr = min(rows, off[i + 1] - r0);
    }
    base += c[i];
  }
  e = __builtin_amdgcn_readlane(ee, src);
  row0 = __builtin_amdgcn_readlane(r0, src);
  mrows = __builtin_amdgcn_readlane(mr, src);
  return true;
}

// the offsets from memory (buffer loads; lanes past E read zeros)
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int E, int rows,
                                          int y, int &e, int &row0, int &mrows) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(offsets, (uint32_t)(E + 1) * 4u);
  int off[kTilePer + 1];
#pragma unroll
  for (int i = 0; i <= kTilePer; ++i)
    off[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(ro, (uint32_t)(kTilePer * lane + i) * 4u, 0, 0);
  return find_tile_from(off, E, rows, y, e, row0, mrows);
}

// GATED: A = gelu_tanh(X Wg^T) * (X Wu^T) -> A [P][N] bf16; else
// Y = A Wd^T -> Y [P][N] bf16.  Tiles of ROWS sorted rows from the tile list.
// KS = 1: the 4 waves take 4 consecutive column groups of NP row tiles, each
// all of K; KS = 4: the 4 waves share one column group and split K (gate/up
// always; down for batches with few tiles, where whole-K streams per wave
// would leave HBM idle).
// PD: K units in flight per wave (deeper for small batches, whose few loads
// are latency-bound and whose occupancy does not matter).
template <int ROWS, int NP, bool GATED, int KS, int FMT, int PD = kGemvPD>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(PD > kGemvPD ? 2 : ROWS == 8 ? 4 : 3)))
void k_expert_gemv(GemvArgs p, const int32_t *__restrict__ offsets, int E, Nvfp4 w0, Nvfp4 w1) {
  constexpr int NW = GATED ? 2 * NP : NP;
  __shared__ __attribute__((aligned(16))) float s_red[KS > 1 ? KS * 64 * NW * 4 : 4];
  const int wave = threadIdx.x >> 6;
  const int nt0 = KS == 1 ? (blockIdx.x * 4 + wave) * NP : blockIdx.x * NP;  // first row tile
  if (nt0 * 16 >= p.N) return;  // past the last column (KS = 4: uniform; KS = 1: no barrier follows)
  int e, row0, mrows;
  if (!find_tile(offsets, E, ROWS, blockIdx.y, e, row0, mrows)) return;  // uniform
  // rows per MFMA block: the smallest packing that holds the tile (uniform)
  if (mrows <= 4) gemv_run<4, NP, GATED, KS, FMT, PD>(p, w0, w1, e, row0, mrows, nt0, s_red);
  else if (ROWS == 8 || mrows <= 8)
    gemv_run<8, NP, GATED, KS, FMT, PD>(p, w0, w1, e, row0, mrows, nt0, s_red);
  else gemv_run<16, NP, GATED, KS, FMT, PD>(p, w0, w1, e, row0, mrows, nt0, s_red);
}

bool tensor_ok(const nvfp4_tensor *t, int E, int N, int K) {
  return t->E == E && t->N == N && t->K == K;
}

// ----------------------------------------------- fused decode layer ----
// For T <= kDecodeMaxT tokens (moe_layer_decode) the selection kernel does
// not run: every workgroup of k_decode_gate_up repeats the top-k selection of
// every token from the logits (a wave per two tokens) and the bucketing of
// the pairs (one wave, in LDS) -- a few microseconds after one load, instead
// of a kernel of its own -- and then runs its gate/up GEMV tile: expert tile
// y (an expert has at most T <= 8 rows: one 8-row tile), column group x.
// Workgroup (0, 0) also writes the routing and bucketing outputs for the
// down projection and the combine.
constexpr int kDecodeMaxT = MOE_DECODE_MAX_TOKENS;
constexpr int kDecodeMaxP = MOE_DECODE_MAX_PAIRS;
static_assert(kDecodeMaxP <= kWave, "the bucketing of the decode layer is one wave's");
static_assert(kDecodeMaxT <= 2 * (kThreads / kWave), "two tokens per selecting wave");
constexpr int kDecodePD = kGemvPD;  // gate/up K units in flight per wave
// gate/up row-tile pairs per wave: 2, or 3 once the grid of 2 would hold
// kDecodeNP3From workgroups or more (most of the 1024 that four per CU keep
// resident at once; 3 pairs per wave keep every tile of a T = 8 batch in one
// round).  Measured, 30-layer sweep at T = 8 1676 -> 1564-1586 us, T = 4 step
// 37.5 -> 36.8 us; at T = 1 (176 workgroups) 3 pairs ran the sweep 673 -> 693 us.
constexpr int kDecodeNP3From = 512;
#ifndef MOE_DECODE_DOWN_PD
#define MOE_DECODE_DOWN_PD 2
#endif
#ifndef MOE_DECODE_NPC
#define MOE_DECODE_NPC 1
#endif
constexpr int kDecodeDownPD = MOE_DECODE_DOWN_PD;  // down K units in flight per wave (fused combine)
constexpr int kDecodeNPC = MOE_DECODE_NPC;          // row tiles per workgroup (fused combine)

struct DecodeRoute {
  const float *logits;  // [T][E]
  const uint16_t *pes;  // [E]
  int T, E;
  int32_t *topk_idx;    // outputs of workgroup (0, 0): [T][top_k]
  float *topk_w, *topk_w_raw;  // topk_w_raw may be null
  int32_t *offsets, *sorted, *rank, *err;  // [E+1], [P], [P], [1]
};

template <int FMT, int NP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void k_decode_gate_up(GemvArgs p, DecodeRoute r, Nvfp4 w0, Nvfp4 w1) {
  constexpr int NW = 2 * NP, KS = 4;
  __shared__ __attribute__((aligned(16))) float s_red[KS * 64 * NW * 4];
  __shared__ int32_t s_idx[kDecodeMaxP], s_sorted[kDecodeMaxP], s_rank[kDecodeMaxP];
  __shared__ float s_w[kDecodeMaxP], s_wr[kDecodeMaxP];
  __shared__ int32_t s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_cnt[kMaxB];
  __shared__ int32_t s_err;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = p.top_k, P = p.P;
  // tokens wave and wave + 4 (T <= 8), the two chains interleaved
  constexpr int NWV = kThreads / kWave;
  if (wave < r.T) {
    if (r.T <= NWV)
      select_token(r.logits, r.pes, wave, r.E, K, s_idx, s_w, s_wr);
    else if (r.E <= 2 * kWave)
      select_tokens_n<2, 2>(r.logits, r.pes, wave, NWV, r.T, r.E, K, s_idx, s_w, s_wr);
    else
      select_tokens_n<MOE_MAX_EXPERTS / kWave, 2>(r.logits, r.pes, wave, NWV, r.T, r.E, K, s_idx,
                                                   s_w, s_wr);
  }
  __syncthreads();
  // One token (uniform): its K selected experts are distinct, so tile y is the
  // y-th smallest selected id, one row at sorted position y -- every
  // workgroup but (0, 0), which writes the routing outputs, skips the
  // bucketing and the tile search.
  const bool one = r.T == 1 && (blockIdx.x | blockIdx.y) != 0;
  if (!one) {
    bucket_one_wave(s_idx, P, r.E, s_off, s_sorted, s_rank, &s_err, s_cnt);
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      for (int i = tid; i < P; i += kThreads) {
        r.topk_idx[i] = s_idx[i];
        r.topk_w[i] = s_w[i];
        if (r.topk_w_raw) r.topk_w_raw[i] = s_wr[i];
        r.sorted[i] = s_sorted[i];
        r.rank[i] = s_rank[i];
      }
      for (int i = tid; i <= r.E; i += kThreads) r.offsets[i] = s_off[i];
      if (tid == 0) *r.err = s_err;
    }
  }
  const int nt0 = blockIdx.x * NP;
  if (nt0 * 16 >= p.N) return;  // uniform: past the last column
  int e, row0, mrows;
  if (one) {
    const int id = lane < K ? s_idx[lane] : 0;
    int below = 0;  // selected ids smaller than this lane's
    for (int jj = 0; jj < K; ++jj) below += s_idx[jj] < id;
    const unsigned long long hit = __ballot(lane < K && below == (int)blockIdx.y);
    if (!hit) return;  // uniform: no tile y
    const int src = (int)__builtin_ctzll(hit);
    e = __builtin_amdgcn_readlane(id, src);
    row0 = (int)blockIdx.y;
    mrows = 1;
    // the pair at sorted position row0 (pair src of token 0), written by
    // every wave before it reads it in the GEMV
    if (lane == 0) s_sorted[row0] = src;
  } else {
    int off[kTilePer + 1];
#pragma unroll
    for (int i = 0; i <= kTilePer; ++i) off[i] = s_off[min(kTilePer * lane + i, r.E)];
    if (!find_tile_from(off, r.E, 8, blockIdx.y, e, row0, mrows)) return;  // uniform
  }
  GemvArgs q = p;
  q.sorted_pairs = s_sorted;
  if (mrows <= 4) gemv_run<4, NP, true, KS, FMT, kDecodePD>(q, w0, w1, e, row0, mrows, nt0, s_red);
  else gemv_run<8, NP, true, KS, FMT, kDecodePD>(q, w0, w1, e, row0, mrows, nt0, s_red);
}

// Down projection and combine of a decode batch in one launch (the plain
// combine of moe_layer_decode, T * top_k <= kDecodeCombineMaxP): workgroup
// (x, t) owns the 16 NPC output columns x of token t, and its wave j the
// token's pair j -- the pair's A row times its expert's down weights over
// all of K (R = 4 packing, one row), rounded to bf16 as Y would be.  The
// waves meet once in LDS and the first 16 NPC threads add the pairs as
// moe_combine does (fp32 fmaf in pair order, one bf16 rounding).  No Y
// round trip and no combine launch; each token's expert weights are read
// once per token (a decode batch of a few tokens shares few experts).
template <int FMT, int NPC>
__global__ __launch_bounds__(kWave * MOE_MAX_TOPK) void k_decode_down_combine(
    GemvArgs p, const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w,
    const int32_t *__restrict__ rank, int E, Nvfp4 d, uint16_t *__restrict__ out) {
  __shared__ float s_y[MOE_MAX_TOPK][16 * NPC];
  const int j = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.y, K = p.top_k;
  const int nt0 = blockIdx.x * NPC;
  const int e = topk_idx[t * K + j], rr = rank[t * K + j];  // uniform per wave
  const bool ok = rr >= 0 && rr < p.P && e >= 0 && e < E;
  float y[NPC];
  if (ok) gemv_run<4, NPC, false, 1, FMT, kDecodeDownPD, false>(p, d, d, e, rr, 1, nt0, nullptr, y);
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) s_y[j][i * 16 + lane] = ok ? y[i] : 0.0f;
  }
  __syncthreads();
  const int c = nt0 * 16 + (int)threadIdx.x;
  if (threadIdx.x < 16 * NPC && c < p.N) {
    float sum = 0.0f;
    for (int jj = 0; jj < K; ++jj) {
      const int q = t * K + jj, r2 = rank[q];
      if (r2 >= 0 && r2 < p.P) sum = fmaf(topk_w[q], s_y[jj][threadIdx.x], sum);
    }
    out[(size_t)t * p.N + c] = f32_to_bf16_rne(sum);
  }
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_workspace_bytes(int32_t T, int32_t top_k, int32_t E, int32_t H, int32_t I) {
  if (T < 0 || top_k <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
  return moe::ws_layout(T, top_k, E, H, I).total;
}

namespace {

using namespace moe;

struct Ws {
  WsLayout L;
  int32_t *x_exp;
  uint32_t *a_max;
  uint16_t *x16, *a, *a16;
};

Ws ws_ptrs(void *workspace, const WsLayout &L) {
  char *ws = (char *)workspace;
  Ws w;
  w.L = L;
  w.x_exp = (int32_t *)(ws + L.x_exp);
  w.a_max = (uint32_t *)(ws + L.a_max);
  w.x16 = (uint16_t *)(ws + L.x16);
  w.a = (uint16_t *)(ws + L.a);
  w.a16 = (uint16_t *)(ws + L.a16);
  return w;
}

// shape / size / workspace checks shared by the expert entry points
int check_common(int32_t T, int32_t top_k, int32_t E, int32_t H, int32_t I, const void *workspace,
                 size_t ws_bytes) {
  if (!workspace) return MOE_ERR_NULL;
  if (T < 0 || top_k <= 0 || H <= 0 || I <= 0 || E <= 0) return MOE_ERR_SHAPE;
  if (H % kCols || I % kCols || E > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOPK)
    return MOE_ERR_UNSUPPORTED;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  // buffer-resource offsets are 32-bit: one expert's tensor and the
  // activation buffers (x16 [T][H], A [P][I]) must stay below 2 GiB
  if ((long long)H * I / 2 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if ((long long)(H > I ? H : I) * T * top_k * 2 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < ws_layout(T, top_k, E, H, I).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// the global scale is read for NVFP4 only
bool tensor_null(const nvfp4_tensor *t) {
  return !t || !t->packed || !t->scales || (t->format == MOE_FORMAT_NVFP4 && !t->global);
}

constexpr int kGemmGateNP = 2;  // tiled mode: gate/up row-tile pairs per wave
constexpr int kGemmDownNP = 4;  // tiled mode: down row tiles per wave

// 1-D grid of the tiled-mode kernels: every (row block, column block), rounded
// up to a multiple of the XCD count (the extra workgroups find no block)
dim3 gemm_grid(int P, int E, int bm, int ncb) {
  const long long tiles = (P + bm - 1) / bm + (E < P ? E : P);  // sum over experts of ceil(M_e / bm)
  const long long n = tiles * ncb;
  return dim3((unsigned)((n + kXcds - 1) / kXcds * kXcds));
}

template <int MSUB, int FMT>
int launch_gate_up(const Ws &w, const int32_t *offsets, const int32_t *sorted_pairs, int T,
                   int top_k, int E, Nvfp4 g, Nvfp4 u, int H, int I, hipStream_t s) {
  constexpr int NP = kGemmGateNP;
  const int ncb = (I + 64 * NP - 1) / (64 * NP);
  MOE_LAUNCH((k_expert_gemm<MSUB, NP, true, FMT>), gemm_grid(T * top_k, E, kBM * MSUB, ncb),
             dim3(kThreads), 0, s,
             (const uint16_t *)w.x16, (const int32_t *)w.x_exp, w.a_max, offsets, sorted_pairs,
             top_k, E, ncb, (uint32_t)((size_t)T * H * 2), g, u, H, I, w.a);
  return MOE_OK;
}

template <int MSUB, int FMT>
int launch_down(const Ws &w, const int32_t *offsets, int T, int top_k, int E, Nvfp4 d, int H,
                int I, uint16_t *y, hipStream_t s) {
  const int ncb = (H + 64 * kGemmDownNP - 1) / (64 * kGemmDownNP);
  const uint16_t *a = w.a;
  if (MSUB == 8) {
    const dim3 grid((T * top_k + 7) / 8);  // 8 rows per workgroup
    if (I <= 8 * 32 * 3)
      MOE_LAUNCH(k_a_f16<3>, grid, dim3(kThreads), 0, s, (const uint16_t *)w.a, w.a_max, T * top_k, I, w.a16);
    else if (I <= 8 * 32 * 8)
      MOE_LAUNCH(k_a_f16<8>, grid, dim3(kThreads), 0, s, (const uint16_t *)w.a, w.a_max, T * top_k, I, w.a16);
    else  // I <= 4096 (gate_up_msub)
      MOE_LAUNCH(k_a_f16<16>, grid, dim3(kThreads), 0, s, (const uint16_t *)w.a, w.a_max, T * top_k, I, w.a16);
    a = w.a16;
  }
  MOE_LAUNCH((k_expert_gemm<MSUB, kGemmDownNP, false, FMT>), gemm_grid(T * top_k, E, kBM * MSUB, ncb),
             dim3(kThreads), 0, s, a, (const int32_t *)nullptr, w.a_max, offsets,
             (const int32_t *)nullptr, top_k, E, ncb, (uint32_t)((size_t)T * top_k * I * 2), d, d,
             I, H, y);
  return MOE_OK;
}

}  // namespace

namespace moe {
int expert_prep_buffers(int T, int top_k, int E, int H, int I, void *workspace, size_t ws_bytes,
                        uint16_t **x16, int32_t **x_exp, uint32_t **a_max) {
  const int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  *x16 = w.x16;
  *x_exp = w.x_exp;
  *a_max = w.a_max;
  return MOE_OK;
}
}  // namespace moe

extern "C" int nvfp4_expert_prep(const uint16_t *x_expert, int32_t T, int32_t top_k, int32_t E,
                                 int32_t H, int32_t I, void *workspace, size_t ws_bytes,
                                 void *stream) {
  if (T > 0 && !x_expert) return MOE_ERR_NULL;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  const int P = T * top_k;
  MOE_LAUNCH(k_prep<false>, dim3((T + 3) / 4), dim3(kThreads), 0, (hipStream_t)stream, x_expert,
             (const uint16_t *)nullptr, 0.0f, T, H, P, w.x16, w.x_exp, w.a_max);
  return MOE_OK;
}

extern "C" int nvfp4_expert_prep_rmsnorm(const uint16_t *x, const uint16_t *norm_weight, float eps,
                                         int32_t T, int32_t top_k, int32_t E, int32_t H,
                                         int32_t I, void *workspace, size_t ws_bytes,
                                         void *stream) {
  if (!norm_weight || (T > 0 && !x)) return MOE_ERR_NULL;
  if (!(eps >= 0.0f)) return MOE_ERR_SHAPE;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  const int P = T * top_k;
  MOE_LAUNCH(k_prep<true>, dim3((T + 3) / 4), dim3(kThreads), 0, (hipStream_t)stream, x,
             norm_weight, eps, T, H, P, w.x16, w.x_exp, w.a_max);
  return MOE_OK;
}

namespace moe {
namespace {

// the gate/up and down launches of one weight format (arguments checked)
template <int FMT>
int gate_up_fmt(const Ws &w, const int32_t *expert_offsets, const int32_t *sorted_pairs, int T,
                int top_k, int E, int H, int I, Nvfp4 g, Nvfp4 u, hipStream_t s) {
  if (gemv_mode(T, top_k, E)) {
    const int rows = gemv_rows(T, top_k, E);
    // the 4 waves of a workgroup split K for one column group of kGateNP row tiles
    const dim3 grid((I + 16 * kGateNP - 1) / (16 * kGateNP), w.L.max_tiles);
    const GemvArgs a{w.x16, w.x_exp, w.a_max, sorted_pairs, top_k, H, I, T * top_k,
                     (uint32_t)((size_t)T * H * 2), w.a};
    if (rows == 8)
      MOE_LAUNCH((k_expert_gemv<8, kGateNP, true, 4, FMT>), grid, dim3(kThreads), 0, s, a,
                 expert_offsets, E, g, u);
    else
      MOE_LAUNCH((k_expert_gemv<16, kGateNP, true, 4, FMT>), grid, dim3(kThreads), 0, s, a,
                 expert_offsets, E, g, u);
    return MOE_OK;
  }
  if (gate_up_msub(T, top_k, E, I) == 8)
    return launch_gate_up<8, FMT>(w, expert_offsets, sorted_pairs, T, top_k, E, g, u, H, I, s);
  return launch_gate_up<4, FMT>(w, expert_offsets, sorted_pairs, T, top_k, E, g, u, H, I, s);
}

template <int FMT>
int down_fmt(const Ws &w, const int32_t *expert_offsets, int T, int top_k, int E, int H, int I,
             Nvfp4 d, uint16_t *y_sorted, hipStream_t s) {
  if (gemv_mode(T, top_k, E)) {
    const int rows = gemv_rows(T, top_k, E);
    // more row tiles per wave halves the activation loads per weight byte
    // but also the waves; it pays once the tiles alone fill the chip
    const bool many = (long long)T * top_k >= 3LL * E;
    const int np = rows == 16 ? kDownNPWide : many ? kDownNPMany : kDownNP;
    const int gx = (H + 64 * np - 1) / (64 * np);
    const bool split = gx * w.L.max_tiles < kGemvSplitBelow;
    const dim3 grid(split ? (H + 16 * np - 1) / (16 * np) : gx, w.L.max_tiles);
    const GemvArgs a{w.a, nullptr, w.a_max, nullptr, top_k, I, H, T * top_k,
                     (uint32_t)((size_t)T * top_k * I * 2), y_sorted};
#define MOE_GEMV_DN(ROWS, NP, KS, ...)                                                          \
  MOE_LAUNCH((k_expert_gemv<ROWS, NP, false, KS, FMT, ##__VA_ARGS__>), grid, dim3(kThreads), 0, s, \
             a, expert_offsets, E, d, d)
    if (rows == 8 && many) {
      if (split) MOE_GEMV_DN(8, kDownNPMany, 4); else MOE_GEMV_DN(8, kDownNPMany, 1);
    } else if (rows == 8) {
      if (split) MOE_GEMV_DN(8, kDownNP, 4); else MOE_GEMV_DN(8, kDownNP, 1);
    } else {
      if (split) MOE_GEMV_DN(16, kDownNPWide, 4); else MOE_GEMV_DN(16, kDownNPWide, 1);
    }
#undef MOE_GEMV_DN
    return MOE_OK;
  }
  if (gate_up_msub(T, top_k, E, I) == 8)
    return launch_down<8, FMT>(w, expert_offsets, T, top_k, E, d, H, I, y_sorted, s);
  return launch_down<4, FMT>(w, expert_offsets, T, top_k, E, d, H, I, y_sorted, s);
}

bool format_known(int f) { return f >= MOE_FORMAT_NVFP4 && f <= MOE_FORMAT_AFF4; }

}  // namespace
}  // namespace moe

extern "C" int nvfp4_expert_gate_up(const nvfp4_tensor *gate, const nvfp4_tensor *up,
                                    const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                    int32_t T, int32_t top_k, int32_t H, int32_t I,
                                    void *workspace, size_t ws_bytes, void *stream) {
  using namespace moe;
  if (tensor_null(gate) || tensor_null(up) || !expert_offsets || (T > 0 && !sorted_pairs))
    return MOE_ERR_NULL;
  const int E = gate->E;
  if (!tensor_ok(gate, E, I, H) || !tensor_ok(up, E, I, H)) return MOE_ERR_SHAPE;
  if (gate->layout != MOE_LAYOUT_TILED || up->layout != MOE_LAYOUT_TILED) return MOE_ERR_UNSUPPORTED;
  if (!format_known(gate->format) || gate->format != up->format) return MOE_ERR_UNSUPPORTED;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  Nvfp4 g{gate->packed, gate->scales, gate->global};
  Nvfp4 u{up->packed, up->scales, up->global};
  hipStream_t s = (hipStream_t)stream;
  switch (gate->format) {
    case MOE_FORMAT_Q4_0:
      return gate_up_fmt<MOE_FORMAT_Q4_0>(w, expert_offsets, sorted_pairs, T, top_k, E, H, I, g, u, s);
    case MOE_FORMAT_AFF4:
      return gate_up_fmt<MOE_FORMAT_AFF4>(w, expert_offsets, sorted_pairs, T, top_k, E, H, I, g, u, s);
    default:
      return gate_up_fmt<MOE_FORMAT_NVFP4>(w, expert_offsets, sorted_pairs, T, top_k, E, H, I, g, u, s);
  }
}

extern "C" int nvfp4_expert_down(const nvfp4_tensor *down, const int32_t *expert_offsets,
                                 int32_t T, int32_t top_k, int32_t H, int32_t I,
                                 uint16_t *y_sorted, void *workspace, size_t ws_bytes,
                                 void *stream) {
  using namespace moe;
  if (tensor_null(down) || !expert_offsets || (T > 0 && !y_sorted)) return MOE_ERR_NULL;
  const int E = down->E;
  if (!tensor_ok(down, E, H, I)) return MOE_ERR_SHAPE;
  if (down->layout != MOE_LAYOUT_TILED || !format_known(down->format)) return MOE_ERR_UNSUPPORTED;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  Nvfp4 d{down->packed, down->scales, down->global};
  hipStream_t s = (hipStream_t)stream;
  switch (down->format) {
    case MOE_FORMAT_Q4_0:
      return down_fmt<MOE_FORMAT_Q4_0>(w, expert_offsets, T, top_k, E, H, I, d, y_sorted, s);
    case MOE_FORMAT_AFF4:
      return down_fmt<MOE_FORMAT_AFF4>(w, expert_offsets, T, top_k, E, H, I, d, y_sorted, s);
    default:
      return down_fmt<MOE_FORMAT_NVFP4>(w, expert_offsets, T, top_k, E, H, I, d, y_sorted, s);
  }
}

extern "C" int nvfp4_expert_mlp(const uint16_t *x_expert, const nvfp4_tensor *gate,
                                const nvfp4_tensor *up, const nvfp4_tensor *down,
                                const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                int32_t T, int32_t top_k, int32_t H, int32_t I,
                                uint16_t *y_sorted, void *workspace, size_t ws_bytes,
                                void *stream) {
  if (tensor_null(gate) || tensor_null(up) || tensor_null(down) || !expert_offsets)
    return MOE_ERR_NULL;
  if (T > 0 && (!x_expert || !sorted_pairs || !y_sorted)) return MOE_ERR_NULL;
  const int E = gate->E;
  if (!tensor_ok(gate, E, I, H) || !tensor_ok(up, E, I, H) || !tensor_ok(down, E, H, I))
    return MOE_ERR_SHAPE;
  if (gate->layout != MOE_LAYOUT_TILED || up->layout != MOE_LAYOUT_TILED ||
      down->layout != MOE_LAYOUT_TILED)
    return MOE_ERR_UNSUPPORTED;
  if (!moe::format_known(gate->format) || gate->format != up->format ||
      !moe::format_known(down->format))
    return MOE_ERR_UNSUPPORTED;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  st = nvfp4_expert_prep(x_expert, T, top_k, E, H, I, workspace, ws_bytes, stream);
  if (st != MOE_OK) return st;
  st = nvfp4_expert_gate_up(gate, up, expert_offsets, sorted_pairs, T, top_k, H, I, workspace,
                            ws_bytes, stream);
  if (st != MOE_OK) return st;
  return nvfp4_expert_down(down, expert_offsets, T, top_k, H, I, y_sorted, workspace, ws_bytes,
                           stream);
}

namespace moe {
// The gate/up stage of the fused decode layer (moe_layer_decode), with the
// top-k selection and the bucketing folded in.  Arguments validated by the
// caller (T <= kDecodeMaxT, T * top_k <= kDecodeMaxP); expert_ws is the
// expert MLP's workspace for (T, top_k, E, H, I), its f16 rows and exponents
// already written and its row maxima cleared.
__attribute__((visibility("hidden"))) int launch_decode_gate_up(
    const float *logits, const uint16_t *pes, int T, int top_k, int E, int H, int I,
    const nvfp4_tensor *gate, const nvfp4_tensor *up, int32_t *topk_idx, float *topk_w,
    float *topk_w_raw, int32_t *offsets, int32_t *sorted, int32_t *rank, int32_t *err,
    void *expert_ws, hipStream_t s) {
  const Ws w = ws_ptrs(expert_ws, ws_layout(T, top_k, E, H, I));
  const int P = T * top_k;
  const GemvArgs a{w.x16, w.x_exp, w.a_max, nullptr, top_k, H, I, P,
                   (uint32_t)((size_t)T * H * 2), w.a};
  const DecodeRoute dr{logits, pes, T, E, topk_idx, topk_w, topk_w_raw, offsets, sorted, rank, err};
  const Nvfp4 g{gate->packed, gate->scales, gate->global}, u{up->packed, up->scales, up->global};
  const int tiles = P < E ? P : E;  // at most one 8-row tile per pair
  const bool np3 = (long long)((I + 31) / 32) * tiles >= kDecodeNP3From;
  const dim3 grid(np3 ? (I + 47) / 48 : (I + 31) / 32, tiles);
#define MOE_DECODE_GU(F)                                                                        \
  if (np3) MOE_LAUNCH((k_decode_gate_up<F, 3>), grid, dim3(kThreads), 0, s, a, dr, g, u);        \
  else MOE_LAUNCH((k_decode_gate_up<F, 2>), grid, dim3(kThreads), 0, s, a, dr, g, u)
  switch (gate->format) {
    case MOE_FORMAT_Q4_0: MOE_DECODE_GU(MOE_FORMAT_Q4_0); break;
    case MOE_FORMAT_AFF4: MOE_DECODE_GU(MOE_FORMAT_AFF4); break;
    default: MOE_DECODE_GU(MOE_FORMAT_NVFP4);
  }
#undef MOE_DECODE_GU
  return MOE_OK;
}

// The down stage and the plain combine of the fused decode layer in one
// launch (T * top_k <= kDecodeCombineMaxP; arguments validated by the
// caller, expert_ws as for launch_decode_gate_up with A written).
__attribute__((visibility("hidden"))) int launch_decode_down_combine(
    const int32_t *topk_idx, const float *topk_w, const int32_t *rank, int T, int top_k, int E,
    int H, int I, const nvfp4_tensor *down, void *expert_ws, uint16_t *out, hipStream_t s) {
  const Ws w = ws_ptrs(expert_ws, ws_layout(T, top_k, E, H, I));
  const int P = T * top_k;
  const GemvArgs a{w.a, nullptr, w.a_max, nullptr, top_k, I, H, P,
                   (uint32_t)((size_t)P * I * 2), nullptr};
  const Nvfp4 d{down->packed, down->scales, down->global};
  const dim3 grid((H + 16 * kDecodeNPC - 1) / (16 * kDecodeNPC), T), block(kWave * top_k);
  switch (down->format) {
    case MOE_FORMAT_Q4_0:
      MOE_LAUNCH((k_decode_down_combine<MOE_FORMAT_Q4_0, kDecodeNPC>), grid, block, 0, s, a,
                 topk_idx, topk_w, rank, E, d, out);
      break;
    case MOE_FORMAT_AFF4:
      MOE_LAUNCH((k_decode_down_combine<MOE_FORMAT_AFF4, kDecodeNPC>), grid, block, 0, s, a,
                 topk_idx, topk_w, rank, E, d, out);
      break;
    default:
      MOE_LAUNCH((k_decode_down_combine<MOE_FORMAT_NVFP4, kDecodeNPC>), grid, block, 0, s, a,
                 topk_idx, topk_w, rank, E, d, out);
  }
  return MOE_OK;
}
}  // namespace moe

// ---- nvfp4_expert_mlp without a caller workspace -------------------------
// For callers that cannot allocate device memory: the workspace is a
// file-scope device array of kStaticScratchBytes, one copy per GPU, which the
// GPU holds until the process ends.  Its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is handed to kernels; the host-side name of the array is not a
// device address.  Every call on a GPU shares that GPU's array.
namespace {
constexpr size_t kStaticScratchBytes = MOE_NOALLOC_MAX_WORKSPACE_BYTES;
constexpr int kStaticMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kStaticMaxDevices] = {};

// the device address of this device's scratch array (nullptr on failure)
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStaticMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int nvfp4_expert_mlp_noalloc(const uint16_t *x_expert, const nvfp4_tensor *gate,
                                        const nvfp4_tensor *up, const nvfp4_tensor *down,
                                        const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                        int32_t T, int32_t top_k, int32_t H, int32_t I,
                                        uint16_t *y_sorted, void *stream) {
  if (tensor_null(gate) || tensor_null(up) || tensor_null(down) || !expert_offsets)
    return MOE_ERR_NULL;
  if (T > 0 && (!x_expert || !sorted_pairs || !y_sorted)) return MOE_ERR_NULL;
  if (T < 0 || top_k <= 0 || H <= 0 || I <= 0) return MOE_ERR_SHAPE;
  const int E = gate->E;
  if (E <= 0) return MOE_ERR_SHAPE;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  const size_t need = moe_workspace_bytes(T, top_k, E, H, I);
  if (need == 0 || need > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
  void *ws = device_scratch();
  if (!ws) return MOE_ERR_LAUNCH;
  return nvfp4_expert_mlp(x_expert, gate, up, down, expert_offsets, sorted_pairs, T, top_k, H, I,
                          y_sorted, ws, kStaticScratchBytes, stream);
}
