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
//       stream, no LDS staging and no barrier in the K loop; activation
//       operands come from transposed copies (16-byte chunks [k/8][row]) so a
//       quarter-wave reads 16 rows of one chunk column.
//     - tiled mode (prefill): 16*MSUB rows per tile staged in LDS per K unit
//       and shared by the 4 waves, weights streamed once per tile.
//    Gate/up epilogue: GELU-tanh gating, A rounded to bf16 (stored transposed
//    in GEMV mode), per-row max|A| by atomicMax on the float bits (an integer
//    max: order-independent).  Down rescales A to f16 by that maximum's power
//    of two and writes Y as bf16 in sorted-row order.
#include "common.h"

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
  size_t x_exp, a_max, x16, a, total;
  int max_tiles;
};

// rows per tile: 16 x MSUB, from the mean bucket size (host-known shapes only)
int choose_msub(int T, int top_k, int E) {
  const long long P = (long long)T * top_k;
  const long long buckets = P < E ? P : E;
  const long long avg = buckets > 0 ? P / buckets : 0;
  if (avg < 24) return 1;
  if (avg < 64) return 2;
  return 4;
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
// [T][H], A [P][I] bf16.
WsLayout ws_layout(int T, int top_k, int E, int H, int I) {
  WsLayout L;
  const size_t P = (size_t)T * top_k;
  const int bm = tile_rows(T, top_k, E);
  L.max_tiles = (int)((P + bm - 1) / bm + (size_t)(E < (int)P ? E : (int)P));
  L.x_exp = 0;
  L.a_max = L.x_exp + moe_align_up((size_t)T * 4, 256);
  L.x16 = L.a_max + moe_align_up(P * 4, 256);
  L.a = L.x16 + moe_align_up((size_t)T * H * 2, 256);
  L.total = L.a + moe_align_up(P * (size_t)I * 2, 256);
  if (L.total < 256) L.total = 256;  // never empty, so T = 0 still gets a valid pointer
  return L;
}

// ---------------------------------------------------------------- prep ----
// Tile `tile` of the list "expert e contributes ceil(M_e / bm) tiles": one
// wave-wide inclusive scan over the bucket sizes; the same answer in every
// lane.  False past the last tile.
__device__ bool find_tile(const int32_t *__restrict__ offsets, int E, int bm, int tile, int &e,
                          int &m0) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < E; base += kWave) {
    const int ee = base + lane;
    const int c = ee < E ? (offsets[ee + 1] - offsets[ee] + bm - 1) / bm : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    // wave-uniform (scalar) values only in the control flow below, so that
    // e and m0 stay scalar after the loop
    const int total = carry + __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1, kWave));
    if (tile < total) {
      const bool hit = tile >= carry + incl - c && tile < carry + incl;
      const unsigned long long mask = __ballot(hit);
      const int src = __ffsll((long long)mask) - 1;
      // the same in every lane: made scalar, so that the buffer resources
      // built from e are uniform (no per-lane descriptor loop)
      e = base + __builtin_amdgcn_readfirstlane(src);
      m0 = __builtin_amdgcn_readfirstlane((tile - carry - __shfl(incl - c, src, kWave)) * bm);
      return true;
    }
    carry = total;
  }
  return false;
}

// One wave per token: row maximum -> exponent -> f16 row scaled by
// 2^(14 - exponent), row-major [T][H]; the other threads clear the per-row
// maximum of A.
__global__ __launch_bounds__(kThreads) void k_prep(const uint16_t *__restrict__ x, int T, int H,
                                                   int P, uint16_t *__restrict__ x16,
                                                   int32_t *__restrict__ x_exp,
                                                   uint32_t *__restrict__ a_max) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = blockIdx.x * kThreads + tid; i < P; i += gridDim.x * kThreads) a_max[i] = 0u;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const uint16_t *row = x + (size_t)t * H;
  float amax = 0.0f;
  for (int k = lane * 8; k < H; k += kWave * 8) {
    const u32x4 v = *(const u32x4 *)(row + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(v[i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(v[i] & 0xFFFF0000u)));
    }
  }
  amax = wave_max(amax);
  const int ex = row_exponent(amax);
  const float f = __builtin_ldexpf(1.0f, 14 - ex);
  for (int k = lane * 8; k < H; k += kWave * 8) {
    const u32x4 v = *(const u32x4 *)(row + k);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16 lo = (f16)(__uint_as_float(v[i] << 16) * f);
      const f16 hi = (f16)(__uint_as_float(v[i] & 0xFFFF0000u) * f);
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *(u32x4 *)(x16 + (size_t)t * H + k) = o;
  }
  if (lane == 0) x_exp[t] = ex;
}

__device__ __forceinline__ float gelu_tanh(float g) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * g * (1.0f + tanhf(c * (g + 0.044715f * g * g * g)));
}

// ------------------------------------------------- grouped expert GEMM ----
// One kernel template for both projections.  A workgroup (4 waves) owns one
// tile of kBM*MSUB sorted rows of one expert and a slice of output columns;
// each wave owns NT row tiles (16 weight rows each) of that slice: for the
// gated projection NT = 2 (16 gate rows and the same 16 up rows), for down
// NT row tiles of consecutive outputs.
//
// K advances in units of 128.  Per unit, the activation tile [rows][128] is
// staged once in LDS as f16 (double-buffered) and shared by the 4 waves; each
// lane loads its 16 bytes of every weight row tile it owns (one contiguous
// kilobyte per wave in the tiled layout), dequantises them in registers and
// runs 4 x MSUB x NT MFMAs 16x16x32.  The weights of the next unit are loaded
// while the current one is multiplied.
constexpr int kUnitK = 128;
constexpr int kLdsRow = kUnitK + 8;  // f16 per LDS row (padding spreads banks)
#ifndef MOE_GEMM_PD
#define MOE_GEMM_PD 1
#endif
constexpr int kPD = MOE_GEMM_PD;     // units in flight per lane (weights and activations)

template <int MSUB, int NT, bool GATED>
__global__ __launch_bounds__(kThreads) void k_expert_gemm(
    const uint16_t *__restrict__ a_src,       // GATED: x16 [T][K] f16; else A [P][K] bf16
    const int32_t *__restrict__ row_exp,      // GATED: x_exp [T];  else unused
    uint32_t *__restrict__ a_max,             // GATED: row max of A (written); else read
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ sorted_pairs, int top_k,
    int E, Nvfp4 w0, Nvfp4 w1,                // GATED: gate, up; else w0 = down
    int K, int N, uint16_t *__restrict__ out, int out_ld) {
  constexpr int BM = kBM * MSUB;
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * kLdsRow];
  __shared__ float s_rowscale[BM];
  int e, m0;
  if (!find_tile(offsets, E, BM, blockIdx.y, e, m0)) return;  // uniform over the workgroup
  const int row0 = offsets[e] + m0;
  const int mrows = min(BM, offsets[e + 1] - row0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nunits = (K + kUnitK - 1) / kUnitK;

  // ---- staging map: thread -> (row, 16-byte column) of the activation tile.
  // Every load below is issued unconditionally from a valid address and the
  // unwanted ones are zeroed with a select, so the loop body has no branches
  // and the compiler can wait for exactly the load it needs (not for all).
  const int st_col = (tid & 15) * 8;  // f16 element offset inside the unit
  const uint16_t *st_src[MSUB];
  bool st_ok[MSUB];
  float st_scale[MSUB];
#pragma unroll
  for (int q = 0; q < MSUB; ++q) {
    const int m = q * kBM + (tid >> 4);
    st_ok[q] = m < mrows;
    st_scale[q] = 1.0f;
    const int mm = st_ok[q] ? m : 0;  // row 0 of the tile always exists
    if (GATED) {
      st_src[q] = a_src + (size_t)(sorted_pairs[row0 + mm] / top_k) * K;
    } else {
      st_src[q] = a_src + (size_t)(row0 + mm) * K;
      st_scale[q] = __builtin_ldexpf(1.0f, 14 - row_exponent(__uint_as_float(a_max[row0 + mm])));
    }
  }
  // per-row factor applied to the fp32 sums: 2^(exponent - 14)
  if (tid < BM) {
    float f = 0.0f;
    if (tid < mrows) {
      const int ex = GATED ? row_exp[sorted_pairs[row0 + tid] / top_k]
                           : row_exponent(__uint_as_float(a_max[row0 + tid]));
      f = __builtin_ldexpf(1.0f, ex - 14);
    }
    s_rowscale[tid] = f;
  }

  auto load_a = [&](int u, u32x4 (&v)[MSUB]) {
    const int k = u * kUnitK + st_col;
    const bool kok = k < K;
    const int kc = kok ? k : 0;
#pragma unroll
    for (int q = 0; q < MSUB; ++q) {
      const u32x4 t = *(const u32x4 *)(st_src[q] + kc);
      const bool ok = kok && st_ok[q];
      v[q] = u32x4{ok ? t[0] : 0u, ok ? t[1] : 0u, ok ? t[2] : 0u, ok ? t[3] : 0u};
    }
  };
  auto store_a = [&](int buf, const u32x4 (&v)[MSUB]) {
#pragma unroll
    for (int q = 0; q < MSUB; ++q) {
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
      *(u32x4 *)(&s_a[buf][(q * kBM + (tid >> 4)) * kLdsRow + st_col]) = o;
    }
  };

  // ---- weight streams of this wave: NT row tiles, read through buffer
  // resources over expert e's tensor: lane (r, g) of unit u is at byte
  // 1024u + 16 lane of its row tile (scales: 128u + 2 lane); lanes past the
  // end of K (and units past the end) read hardware zeros.
  __amdgpu_buffer_rsrc_t rw[NT], rs[NT];
  uint32_t vw[NT], vs[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const Nvfp4 &w = (GATED && i == 1) ? w1 : w0;
    const int nt = GATED ? (blockIdx.x * 4 + wave) : ((blockIdx.x * 4 + wave) * NT + i);
    rw[i] = make_rsrc(w.packed + (size_t)e * N * (K / 2), (uint32_t)((size_t)N * (K / 2)));
    rs[i] = make_rsrc(w.scales + (size_t)e * N * (K / 16), (uint32_t)((size_t)N * (K / 16)));
    vw[i] = (uint32_t)nt * 16 * (K / 2) + lane * 16;
    vs[i] = (uint32_t)nt * K + lane * 2;
  }
  auto load_w = [&](int u, u32x4 (&wv)[NT], uint32_t (&sv)[NT]) {
    const bool ok = u < nunits && u * kUnitK + 32 * g < K;
    const uint32_t ow = ok ? (uint32_t)u * 1024 : kOOB, os = ok ? (uint32_t)u * 128 : kOOB;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      wv[i] = bload16_nt(rw[i], vw[i] + ow);
      sv[i] = bload2(rs[i], vs[i] + os);
    }
  };

  f32x4 acc[MSUB][NT];
#pragma unroll
  for (int q = 0; q < MSUB; ++q)
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[q][i] = f32x4{0, 0, 0, 0};

  // ---- pipeline.  Weights: unit u+kPD is loaded into the register slot
  // that unit u just used.  Activations: unit u+kPD is loaded into a
  // register slot before unit u is multiplied and reaches LDS (double
  // buffer) at the end of iteration u+kPD-1.  Units past the end are zeros
  // (the unit count is rounded up to a multiple of kPD).  One barrier per unit.
  u32x4 wbuf[kPD][NT];
  uint32_t sbuf[kPD][NT];
  u32x4 av[kPD][MSUB];
  load_a(0, av[0]);
  store_a(0, av[0]);
#pragma unroll
  for (int d = 1; d < kPD; ++d) load_a(d, av[d]);
#pragma unroll
  for (int d = 0; d < kPD; ++d) load_w(d, wbuf[d], sbuf[d]);
  __syncthreads();

  const int nu = (nunits + kPD - 1) / kPD * kPD;
  for (int u0 = 0; u0 < nu; u0 += kPD) {
#pragma unroll
    for (int d = 0; d < kPD; ++d) {
      const int u = u0 + d;
      load_a(u + kPD, av[d]);
      const uint16_t *abuf = s_a[u & 1];
      f16x2 bs[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) bs[i] = block_scales_f16(sbuf[d][i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f16x8 b[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) b[i] = dequant8(wbuf[d][i][j], bs[i][j >> 1]);
#pragma unroll
        for (int q = 0; q < MSUB; ++q) {
          const f16x8 a = __builtin_bit_cast(
              f16x8, *(const u32x4 *)(abuf + (q * kBM + r) * kLdsRow + 32 * g + 8 * j));
#pragma unroll
          for (int i = 0; i < NT; ++i) acc[q][i] = mfma16x16x32(a, b[i], acc[q][i]);
        }
      }
      load_w(u + kPD, wbuf[d], sbuf[d]);
      store_a((u + 1) & 1, av[(d + 1) % kPD]);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds rows 16q + 4g + jj, column r of each row tile
  const int e_global = e;
  if (GATED) {
    const float gg = w0.global[e_global], gu = w1.global[e_global];
    const int col = (blockIdx.x * 4 + wave) * 16 + r;
#pragma unroll
    for (int q = 0; q < MSUB; ++q) {
      float rmax[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m = q * kBM + 4 * g + jj;
        rmax[jj] = 0.0f;
        if (m < mrows) {
          const float f = s_rowscale[m];
          const float G = acc[q][0][jj] * (gg * f), U = acc[q][1][jj] * (gu * f);
          const uint16_t ab = f32_to_bf16(gelu_tanh(G) * U);
          out[(size_t)(row0 + m) * out_ld + col] = ab;
          rmax[jj] = fabsf(bf16_to_f32(ab));
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) rmax[jj] = fmaxf(rmax[jj], __shfl_xor(rmax[jj], o, kWave));
        const int m = q * kBM + 4 * g + jj;
        if (r == 0 && m < mrows)
          atomicMax(&a_max[row0 + m], __float_as_uint(rmax[jj]));
      }
    }
  } else {
    const float gd = w0.global[e_global];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int col = ((blockIdx.x * 4 + wave) * NT + i) * 16 + r;
#pragma unroll
      for (int q = 0; q < MSUB; ++q)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int m = q * kBM + 4 * g + jj;
          if (m < mrows)
            out[(size_t)(row0 + m) * out_ld + col] = f32_to_bf16(acc[q][i][jj] * (gd * s_rowscale[m]));
        }
    }
  }
}

// ------------------------------------------------------- GEMV mode ----
// Few rows per expert (decode).  Every wave is an independent stream: no LDS
// staging and no barrier in the K loop.  A wave owns NW weight row tiles
// (gated: NP gate tiles and the same NP up tiles; down: NP tiles) of one
// tile of up to 4 * NGMAX sorted rows of one expert, processed as groups of 4
// rows.
//
// Four rows fill one 16x16x32 MFMA block-diagonally, so that one 16-byte
// load per lane brings 4 rows x 128 K of activations per K unit: lane
// (r, g) loads row 4q + r%4 of group q, K = 128u + 32g + 8h .. +7 with
// h = r/4, and feeds it to MFMA h only (zeros to the other three).  MFMA j
// multiplies by dword j of the lane's weight bytes (K = 128u + 32g + 8j), so
// accumulator row 4h + m holds row m's dot product over the K chunks with
// j = h; the four partial rows of a row are summed once after the K loop.
// Units up to kGemvPD ahead are in flight.
constexpr int kGemvPD = 2;
constexpr int kGateNP = 2;  // gate/up row-tile pairs per wave
constexpr int kDownNP = 4;  // down row tiles per wave

template <int NG, int NW>
struct GemvUnit {
  u32x4 a[NG];
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

template <int NG, int NP, bool GATED>
__device__ __forceinline__ void gemv_run(const GemvArgs &p, const Nvfp4 &w0, const Nvfp4 &w1,
                                         int e, int row0, int mrows, int nt0) {
  constexpr int NW = GATED ? 2 * NP : NP;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4, h = r >> 2, m4 = r & 3;
  const int K = p.K, N = p.N;
  const int nunits = (K + kUnitK - 1) / kUnitK;

  // activation rows of this lane (one per group) and their offsets
  uint32_t va[NG];
  float a_scale[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int m = 4 * q + m4;
    const bool ok = m < mrows;
    const int prow = ok ? row0 + m : row0;
    const int arow = GATED ? p.sorted_pairs[prow] / p.top_k : prow;
    va[q] = ok ? (uint32_t)arow * (uint32_t)K * 2 + (uint32_t)(32 * g + 8 * h) * 2 : kOOB;
    a_scale[q] = 1.0f;
    if (!GATED) a_scale[q] = __builtin_ldexpf(1.0f, 14 - row_exponent(__uint_as_float(p.a_max[prow])));
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a_src, p.a_bytes);

  // weight streams: expert e's tensors through buffer resources; offsets past
  // the end (lanes past K, units past the end) read hardware zeros
  __amdgpu_buffer_rsrc_t rw[NW], rs[NW];
  uint32_t vw[NW], vs[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const Nvfp4 &w = (GATED && i >= NP) ? w1 : w0;
    const int nt = nt0 + (GATED ? i % NP : i);
    rw[i] = make_rsrc(w.packed + (size_t)e * N * (K / 2), (uint32_t)((size_t)N * (K / 2)));
    rs[i] = make_rsrc(w.scales + (size_t)e * N * (K / 16), (uint32_t)((size_t)N * (K / 16)));
    vw[i] = (uint32_t)nt * 16 * (K / 2) + lane * 16;
    vs[i] = (uint32_t)nt * K + lane * 2;
  }
  auto load = [&](int u, GemvUnit<NG, NW> &d) {
    const bool kok = u < nunits && u * kUnitK + 32 * g < K;
    const uint32_t ow = kok ? (uint32_t)u * 1024 : kOOB, os = kok ? (uint32_t)u * 128 : kOOB;
    // va[q] is kOOB for rows past the tile; kOOB + 256u stays out of range
#pragma unroll
    for (int q = 0; q < NG; ++q) d.a[q] = bload16(ra, kok ? va[q] + (uint32_t)u * kUnitK * 2 : kOOB);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      d.w[i] = bload16_nt(rw[i], vw[i] + ow);
      d.s[i] = bload2(rs[i], vs[i] + os);
    }
  };

  f32x4 acc[NG][NW];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int i = 0; i < NW; ++i) acc[q][i] = f32x4{0, 0, 0, 0};
  auto compute = [&](const GemvUnit<NG, NW> &c) {
    f16x8 a[NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      if (GATED) {
        a[q] = __builtin_bit_cast(f16x8, c.a[q]);
      } else {  // bf16 -> f16 with the row's power of two (exact)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          a[q][2 * t] = (f16)(__uint_as_float(c.a[q][t] << 16) * a_scale[q]);
          a[q][2 * t + 1] = (f16)(__uint_as_float(c.a[q][t] & 0xFFFF0000u) * a_scale[q]);
        }
      }
    }
    f16x2 bs[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) bs[i] = block_scales_f16(c.s[i]);
    const f16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 b[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) b[i] = dequant8(c.w[i][j], bs[i][j >> 1]);
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        const f16x8 aj = h == j ? a[q] : zero;
#pragma unroll
        for (int i = 0; i < NW; ++i) acc[q][i] = mfma16x16x32(aj, b[i], acc[q][i]);
      }
    }
  };

  // ---- K loop: kGemvPD + 1 register buffers.  The loads of unit u + kGemvPD
  // are issued before unit u is multiplied (a scheduling barrier keeps them
  // there), so kGemvPD units stay in flight while a wave computes.  The unit
  // count is rounded up to a multiple of the buffer count; the extra units
  // read zeros through the buffer range check and add nothing.
  constexpr int NB = kGemvPD + 1;
  GemvUnit<NG, NW> buf[NB];
#pragma unroll
  for (int d = 0; d < kGemvPD; ++d) load(d, buf[d]);
  const int nu = (nunits + NB - 1) / NB * NB;
  for (int u0 = 0; u0 < nu; u0 += NB) {
#pragma unroll
    for (int d = 0; d < NB; ++d) {
      load(u0 + d + kGemvPD, buf[(d + kGemvPD) % NB]);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- sum the four partial rows: lane (n, g) holds accumulator rows
  // 4g + jj, i.e. partial h = g of row jj; after the butterfly every lane
  // holds the full sums and lane (n, g) keeps row 4q + g.
  float v[NG][NW];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      float s4[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float t = acc[q][i][jj];
        t += __shfl_xor(t, 16, kWave);
        t += __shfl_xor(t, 32, kWave);
        s4[jj] = t;
      }
      v[q][i] = g == 0 ? s4[0] : g == 1 ? s4[1] : g == 2 ? s4[2] : s4[3];
    }

  if (GATED) {
    const float gg = w0.global[e], gu = w1.global[e];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int m = 4 * q + g;
      const bool ok = m < mrows;
      float f = 0.0f;
      if (ok) f = __builtin_ldexpf(1.0f, p.x_exp[p.sorted_pairs[row0 + m] / p.top_k] - 14);
      float rmax = 0.0f;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const float G = v[q][i] * (gg * f), U = v[q][NP + i] * (gu * f);
        const uint16_t ab = f32_to_bf16(gelu_tanh(G) * U);
        if (ok) p.out[(size_t)(row0 + m) * N + (nt0 + i) * 16 + r] = ab;
        rmax = fmaxf(rmax, ok ? fabsf(bf16_to_f32(ab)) : 0.0f);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o, kWave));
      if (r == 0 && ok) atomicMax(&p.a_max[row0 + m], __float_as_uint(rmax));
    }
  } else {
    const float gd = w0.global[e];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int m = 4 * q + g;
      if (m < mrows) {
        const float f =
            gd * __builtin_ldexpf(1.0f, row_exponent(__uint_as_float(p.a_max[row0 + m])) - 14);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int n = (nt0 + i) * 16 + r;
          if (n < N) p.out[(size_t)(row0 + m) * N + n] = f32_to_bf16(v[q][i] * f);
        }
      }
    }
  }
}

// GATED: A = gelu_tanh(X Wg^T) * (X Wu^T) -> A [P][N] bf16; else
// Y = A Wd^T -> Y [P][N] bf16.  Tiles of ROWS sorted rows.
template <int ROWS, int NP, bool GATED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(ROWS == 8 ? 3 : 2)))
void k_expert_gemv(GemvArgs p, const int32_t *__restrict__ offsets,
                                                          int E, Nvfp4 w0, Nvfp4 w1) {
  const int wave = threadIdx.x >> 6;
  const int nt0 = (blockIdx.x * 4 + wave) * NP;  // first output row tile of this wave
  if (nt0 * 16 >= p.N) return;                   // past the last column (no barrier follows)
  int e, m0;
  if (!find_tile(offsets, E, ROWS, blockIdx.y, e, m0)) return;
  const int row0 = offsets[e] + m0;
  const int mrows = min(ROWS, offsets[e + 1] - row0);
  const int ng = (mrows + 3) >> 2;  // uniform over the workgroup
  if (ROWS == 8) {
    if (ng <= 1) gemv_run<1, NP, GATED>(p, w0, w1, e, row0, mrows, nt0);
    else gemv_run<2, NP, GATED>(p, w0, w1, e, row0, mrows, nt0);
  } else {
    if (ng <= 1) gemv_run<1, NP, GATED>(p, w0, w1, e, row0, mrows, nt0);
    else if (ng == 2) gemv_run<2, NP, GATED>(p, w0, w1, e, row0, mrows, nt0);
    else gemv_run<4, NP, GATED>(p, w0, w1, e, row0, mrows, nt0);
  }
}

bool tensor_ok(const nvfp4_tensor *t, int E, int N, int K) {
  return t->E == E && t->N == N && t->K == K;
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
  uint16_t *x16, *a;
};

Ws ws_ptrs(void *workspace, const WsLayout &L) {
  char *ws = (char *)workspace;
  Ws w;
  w.L = L;
  w.x_exp = (int32_t *)(ws + L.x_exp);
  w.a_max = (uint32_t *)(ws + L.a_max);
  w.x16 = (uint16_t *)(ws + L.x16);
  w.a = (uint16_t *)(ws + L.a);
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
  // transposed activations must stay below 2 GiB
  if ((long long)H * I / 2 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (gemv_mode(T, top_k, E) && (long long)(H > I ? H : I) * T * top_k * 2 >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < ws_layout(T, top_k, E, H, I).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

bool tensor_null(const nvfp4_tensor *t) { return !t || !t->packed || !t->scales || !t->global; }

template <int MSUB>
int launch_gate_up(const Ws &w, const int32_t *offsets, const int32_t *sorted_pairs, int top_k,
                   int E, Nvfp4 g, Nvfp4 u, int H, int I, hipStream_t s) {
  MOE_LAUNCH((k_expert_gemm<MSUB, 2, true>), dim3(I / kCols, w.L.max_tiles), dim3(kThreads), 0, s,
             (const uint16_t *)w.x16, (const int32_t *)w.x_exp, w.a_max, offsets, sorted_pairs,
             top_k, E, g, u, H, I, w.a, I);
  return MOE_OK;
}

template <int MSUB, int NT>
int launch_down(const Ws &w, const int32_t *offsets, int top_k, int E, Nvfp4 d, int H, int I,
                uint16_t *y, hipStream_t s) {
  MOE_LAUNCH((k_expert_gemm<MSUB, NT, false>), dim3(H / (kCols * NT), w.L.max_tiles),
             dim3(kThreads), 0, s, (const uint16_t *)w.a, (const int32_t *)nullptr, w.a_max,
             offsets, (const int32_t *)nullptr, top_k, E, d, d, I, H, y, H);
  return MOE_OK;
}

}  // namespace

extern "C" int nvfp4_expert_prep(const uint16_t *x_expert, int32_t T, int32_t top_k, int32_t E,
                                 int32_t H, int32_t I, void *workspace, size_t ws_bytes,
                                 void *stream) {
  if (T > 0 && !x_expert) return MOE_ERR_NULL;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  const int P = T * top_k;
  MOE_LAUNCH(k_prep, dim3((T + 3) / 4), dim3(kThreads), 0, (hipStream_t)stream, x_expert, T, H,
             P, w.x16, w.x_exp, w.a_max);
  return MOE_OK;
}

extern "C" int nvfp4_expert_gate_up(const nvfp4_tensor *gate, const nvfp4_tensor *up,
                                    const int32_t *expert_offsets, const int32_t *sorted_pairs,
                                    int32_t T, int32_t top_k, int32_t H, int32_t I,
                                    void *workspace, size_t ws_bytes, void *stream) {
  if (tensor_null(gate) || tensor_null(up) || !expert_offsets || (T > 0 && !sorted_pairs))
    return MOE_ERR_NULL;
  const int E = gate->E;
  if (!tensor_ok(gate, E, I, H) || !tensor_ok(up, E, I, H)) return MOE_ERR_SHAPE;
  if (gate->layout != MOE_LAYOUT_TILED || up->layout != MOE_LAYOUT_TILED) return MOE_ERR_UNSUPPORTED;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  Nvfp4 g{gate->packed, gate->scales, gate->global};
  Nvfp4 u{up->packed, up->scales, up->global};
  hipStream_t s = (hipStream_t)stream;
  if (gemv_mode(T, top_k, E)) {
    const int cols = 4 * 16 * kGateNP;  // output columns per workgroup
    const dim3 grid((I + cols - 1) / cols, w.L.max_tiles);
    const GemvArgs a{w.x16, w.x_exp, w.a_max, sorted_pairs, top_k, H, I, T * top_k,
                     (uint32_t)((size_t)T * H * 2), w.a};
    if (gemv_rows(T, top_k, E) == 8)
      MOE_LAUNCH((k_expert_gemv<8, kGateNP, true>), grid, dim3(kThreads), 0, s, a, expert_offsets, E, g, u);
    else
      MOE_LAUNCH((k_expert_gemv<16, kGateNP, true>), grid, dim3(kThreads), 0, s, a, expert_offsets, E, g, u);
    return MOE_OK;
  }
  switch (choose_msub(T, top_k, E)) {
    case 1: return launch_gate_up<1>(w, expert_offsets, sorted_pairs, top_k, E, g, u, H, I, s);
    case 2: return launch_gate_up<2>(w, expert_offsets, sorted_pairs, top_k, E, g, u, H, I, s);
    default: return launch_gate_up<4>(w, expert_offsets, sorted_pairs, top_k, E, g, u, H, I, s);
  }
}

extern "C" int nvfp4_expert_down(const nvfp4_tensor *down, const int32_t *expert_offsets,
                                 int32_t T, int32_t top_k, int32_t H, int32_t I,
                                 uint16_t *y_sorted, void *workspace, size_t ws_bytes,
                                 void *stream) {
  if (tensor_null(down) || !expert_offsets || (T > 0 && !y_sorted)) return MOE_ERR_NULL;
  const int E = down->E;
  if (!tensor_ok(down, E, H, I)) return MOE_ERR_SHAPE;
  if (down->layout != MOE_LAYOUT_TILED) return MOE_ERR_UNSUPPORTED;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  Nvfp4 d{down->packed, down->scales, down->global};
  hipStream_t s = (hipStream_t)stream;
  if (gemv_mode(T, top_k, E)) {
    const int cols = 4 * 16 * kDownNP;
    const dim3 grid((H + cols - 1) / cols, w.L.max_tiles);
    const GemvArgs a{w.a, nullptr, w.a_max, nullptr, top_k, I, H, T * top_k,
                     (uint32_t)((size_t)T * top_k * I * 2), y_sorted};
    if (gemv_rows(T, top_k, E) == 8)
      MOE_LAUNCH((k_expert_gemv<8, kDownNP, false>), grid, dim3(kThreads), 0, s, a, expert_offsets, E, d, d);
    else
      MOE_LAUNCH((k_expert_gemv<16, kDownNP, false>), grid, dim3(kThreads), 0, s, a, expert_offsets, E, d, d);
    return MOE_OK;
  }
  const bool two = H % (2 * kCols) == 0;
  switch (choose_msub(T, top_k, E)) {
    case 1: return two ? launch_down<1, 2>(w, expert_offsets, top_k, E, d, H, I, y_sorted, s)
                       : launch_down<1, 1>(w, expert_offsets, top_k, E, d, H, I, y_sorted, s);
    case 2: return two ? launch_down<2, 2>(w, expert_offsets, top_k, E, d, H, I, y_sorted, s)
                       : launch_down<2, 1>(w, expert_offsets, top_k, E, d, H, I, y_sorted, s);
    default: return two ? launch_down<4, 2>(w, expert_offsets, top_k, E, d, H, I, y_sorted, s)
                        : launch_down<4, 1>(w, expert_offsets, top_k, E, d, H, I, y_sorted, s);
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
