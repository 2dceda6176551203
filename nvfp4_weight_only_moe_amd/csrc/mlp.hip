// nvfp4_expert_mlp: the routed experts of the Gemma-4 MoE block on gfx950.
//
// Per expert e and its bucket of rows X_e ("Gemma 4 26B-A4B (MoE) - Core AI",
// Architecture: GELU-gated experts, gelu_pytorch_tanh; gate/up 2816 -> 704,
// down 704 -> 2816):
//     A = gelu_tanh(X_e Wg^T) * (X_e Wu^T),   Y = A Wd^T
// with W = E2M1 x E4M3 block scale x FP32 tensor scale ("Gemma-4-26B-A4B-
// NVFP4-mlx", Notes).
//
// Three kernels:
//  * prep: per token, the exponent of max|x| and the f16 copy of the row
//    scaled by 2^(14 - exponent) (exact for every bf16 value down to 2^-29 of
//    the row maximum); the list of (expert, first row) tiles of kBM rows; the
//    per-row max of A cleared.
//  * gate/up: one workgroup = one tile x 64 output columns; each wave owns 16
//    columns of gate and the same 16 of up.  Lane (r, g) of a wave streams 32
//    consecutive K elements of weight row n0 + r per step (one 16-byte load of
//    packed nibbles + two block-scale bytes), dequantises them in registers
//    (hardware FP4->f16 conversion with the block scale's power of two, one
//    packed f16 multiply by its mantissa) and feeds four f16 MFMAs 16x16x32.
//    Which 32 K indices a lane owns is free as long as the activation operand
//    uses the same map, so every load is a contiguous 16 bytes.  Epilogue:
//    tensor scale and row power of two on the fp32 sums, GELU-tanh gating,
//    A stored as bf16 in sorted-row order, per-row max|A| by atomicMax on the
//    float bits (integer max: order-independent).
//  * down: the tile's A rows are rescaled to f16 into LDS once; the same
//    streaming loop over the down rows; Y stored as bf16.
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
  size_t hdr, tiles, x_exp, a_max, x16, a, total;
  int max_tiles;
};

WsLayout ws_layout(int T, int top_k, int E, int H, int I) {
  WsLayout L;
  const size_t P = (size_t)T * top_k;
  L.max_tiles = (int)((P + kBM - 1) / kBM + (size_t)(E < (int)P ? E : (int)P));
  L.hdr = 0;
  L.tiles = 256;
  L.x_exp = L.tiles + moe_align_up((size_t)L.max_tiles * 8 + 8, 256);
  L.a_max = L.x_exp + moe_align_up((size_t)T * 4, 256);
  L.x16 = L.a_max + moe_align_up(P * 4, 256);
  L.a = L.x16 + moe_align_up((size_t)T * H * 2, 256);
  L.total = L.a + moe_align_up(P * (size_t)I * 2, 256);
  return L;
}

// ---------------------------------------------------------------- prep ----
__global__ __launch_bounds__(kThreads) void k_prep(const uint16_t *__restrict__ x, int T, int H,
                                                   const int32_t *__restrict__ offsets, int E,
                                                   int P, int bm, uint16_t *__restrict__ x16,
                                                   int32_t *__restrict__ x_exp,
                                                   int32_t *__restrict__ tiles,
                                                   int32_t *__restrict__ ntiles,
                                                   uint32_t *__restrict__ a_max) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (blockIdx.x == gridDim.x - 1) {
    // tile list: expert e contributes ceil(M_e / bm) tiles (wave 0 only)
    if (wave != 0) return;
    int carry = 0;
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const int m = e < E ? offsets[e + 1] - offsets[e] : 0;
      const int c = (m + bm - 1) / bm;
      int incl = c;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
      }
      for (int i = 0; i < c; ++i) {
        tiles[2 * (carry + incl - c + i)] = e;
        tiles[2 * (carry + incl - c + i) + 1] = i * bm;
      }
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) ntiles[0] = carry;
    return;
  }
  // clear the per-row max of A
  for (int i = blockIdx.x * kThreads + tid; i < P; i += (gridDim.x - 1) * kThreads) a_max[i] = 0u;
  // one wave per token row
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
  uint16_t *out = x16 + (size_t)t * H;
  for (int k = lane * 8; k < H; k += kWave * 8) {
    const u32x4 v = *(const u32x4 *)(row + k);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16 lo = (f16)(__uint_as_float(v[i] << 16) * f);
      const f16 hi = (f16)(__uint_as_float(v[i] & 0xFFFF0000u) * f);
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *(u32x4 *)(out + k) = o;
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
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    Nvfp4 w0, Nvfp4 w1,                       // GATED: gate, up; else w0 = down
    int K, int N, uint16_t *__restrict__ out, int out_ld) {
  constexpr int BM = kBM * MSUB;
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * kLdsRow];
  __shared__ float s_rowscale[BM];
  const int tile = blockIdx.y;
  if (tile >= ntiles[0]) return;
  const int e = tiles[2 * tile], m0 = tiles[2 * tile + 1];
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

  // ---- weight streams of this wave: NT row tiles.  Lane (r, g) of unit u
  // is at +1024u (packed) / +128u (scales); lane (r, 0) of unit 0 always
  // exists and stands in for lanes past the end of K.
  const uint8_t *wp[NT];
  const uint8_t *ws[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const Nvfp4 &w = (GATED && i == 1) ? w1 : w0;
    const int nt = GATED ? (blockIdx.x * 4 + wave) : ((blockIdx.x * 4 + wave) * NT + i);
    wp[i] = w.packed + (size_t)e * N * (K / 2) + (size_t)nt * 16 * (K / 2) + lane * 16;
    ws[i] = w.scales + (size_t)e * N * (K / 16) + (size_t)nt * K + lane * 2;
  }
  auto load_w = [&](int u, u32x4 (&wv)[NT], uint32_t (&sv)[NT]) {
    const bool ok = u < nunits && u * kUnitK + 32 * g < K;
    const size_t po = ok ? (size_t)u * 1024 : 0, so = ok ? (size_t)u * 128 : 0;
    const int pb = ok ? 0 : 256 * g, sb = ok ? 0 : 32 * g;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const u32x4 t = __builtin_nontemporal_load((const u32x4 *)(wp[i] + po - pb));
      const uint32_t c = *(const uint16_t *)(ws[i] + so - sb);
      wv[i] = u32x4{ok ? t[0] : 0u, ok ? t[1] : 0u, ok ? t[2] : 0u, ok ? t[3] : 0u};
      sv[i] = ok ? c : 0u;
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
      BlockScale bs[NT][2];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        bs[i][0] = decode_block_scale(sbuf[d][i] & 0xFF);
        bs[i][1] = decode_block_scale(sbuf[d][i] >> 8);
      }
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
  int32_t *tiles, *ntiles, *x_exp;
  uint32_t *a_max;
  uint16_t *x16, *a;
};

Ws ws_ptrs(void *workspace, const WsLayout &L) {
  char *ws = (char *)workspace;
  Ws w;
  w.L = L;
  w.tiles = (int32_t *)(ws + L.tiles);
  w.ntiles = (int32_t *)(ws + L.hdr) + 1;
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
  if (ws_bytes < ws_layout(T, top_k, E, H, I).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

bool tensor_null(const nvfp4_tensor *t) { return !t || !t->packed || !t->scales || !t->global; }

// rows per tile: 16 x MSUB, from the mean bucket size (host-known shapes only)
int choose_msub(int T, int top_k, int E) {
  const long long P = (long long)T * top_k;
  const long long buckets = P < E ? P : E;
  const long long avg = buckets > 0 ? P / buckets : 0;
  if (avg < 24) return 1;
  if (avg < 64) return 2;
  return 4;
}

template <int MSUB>
int launch_gate_up(const Ws &w, const int32_t *offsets, const int32_t *sorted_pairs, int top_k,
                   Nvfp4 g, Nvfp4 u, int H, int I, hipStream_t s) {
  MOE_LAUNCH((k_expert_gemm<MSUB, 2, true>), dim3(I / kCols, w.L.max_tiles), dim3(kThreads), 0, s,
             (const uint16_t *)w.x16, (const int32_t *)w.x_exp, w.a_max, offsets, sorted_pairs,
             top_k, (const int32_t *)w.tiles, (const int32_t *)w.ntiles, g, u, H, I, w.a, I);
  return MOE_OK;
}

template <int MSUB, int NT>
int launch_down(const Ws &w, const int32_t *offsets, int top_k, Nvfp4 d, int H, int I,
                uint16_t *y, hipStream_t s) {
  MOE_LAUNCH((k_expert_gemm<MSUB, NT, false>), dim3(H / (kCols * NT), w.L.max_tiles),
             dim3(kThreads), 0, s, (const uint16_t *)w.a, (const int32_t *)nullptr, w.a_max,
             offsets, (const int32_t *)nullptr, top_k, (const int32_t *)w.tiles,
             (const int32_t *)w.ntiles, d, d, I, H, y, H);
  return MOE_OK;
}

}  // namespace

extern "C" int nvfp4_expert_prep(const uint16_t *x_expert, const int32_t *expert_offsets,
                                 int32_t T, int32_t top_k, int32_t E, int32_t H, int32_t I,
                                 void *workspace, size_t ws_bytes, void *stream) {
  if (!expert_offsets || (T > 0 && !x_expert)) return MOE_ERR_NULL;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  const int bm = kBM * choose_msub(T, top_k, E);
  MOE_LAUNCH(k_prep, dim3((T + 3) / 4 + 1), dim3(kThreads), 0, (hipStream_t)stream,
             x_expert, T, H, expert_offsets, E, T * top_k, bm, w.x16, w.x_exp, w.tiles,
             w.ntiles, w.a_max);
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
  switch (choose_msub(T, top_k, E)) {
    case 1: return launch_gate_up<1>(w, expert_offsets, sorted_pairs, top_k, g, u, H, I, s);
    case 2: return launch_gate_up<2>(w, expert_offsets, sorted_pairs, top_k, g, u, H, I, s);
    default: return launch_gate_up<4>(w, expert_offsets, sorted_pairs, top_k, g, u, H, I, s);
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
  const bool two = H % (2 * kCols) == 0;
  switch (choose_msub(T, top_k, E)) {
    case 1: return two ? launch_down<1, 2>(w, expert_offsets, top_k, d, H, I, y_sorted, s)
                       : launch_down<1, 1>(w, expert_offsets, top_k, d, H, I, y_sorted, s);
    case 2: return two ? launch_down<2, 2>(w, expert_offsets, top_k, d, H, I, y_sorted, s)
                       : launch_down<2, 1>(w, expert_offsets, top_k, d, H, I, y_sorted, s);
    default: return two ? launch_down<4, 2>(w, expert_offsets, top_k, d, H, I, y_sorted, s)
                        : launch_down<4, 1>(w, expert_offsets, top_k, d, H, I, y_sorted, s);
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
  st = nvfp4_expert_prep(x_expert, expert_offsets, T, top_k, E, H, I, workspace, ws_bytes, stream);
  if (st != MOE_OK) return st;
  st = nvfp4_expert_gate_up(gate, up, expert_offsets, sorted_pairs, T, top_k, H, I, workspace,
                            ws_bytes, stream);
  if (st != MOE_OK) return st;
  return nvfp4_expert_down(down, expert_offsets, T, top_k, H, I, y_sorted, workspace, ws_bytes,
                           stream);
}
