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
                                                   int P, uint16_t *__restrict__ x16,
                                                   int32_t *__restrict__ x_exp,
                                                   int32_t *__restrict__ tiles,
                                                   int32_t *__restrict__ ntiles,
                                                   uint32_t *__restrict__ a_max) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (blockIdx.x == gridDim.x - 1) {
    // tile list: expert e contributes ceil(M_e / kBM) tiles (wave 0 only)
    if (wave != 0) return;
    int carry = 0;
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const int m = e < E ? offsets[e + 1] - offsets[e] : 0;
      const int c = (m + kBM - 1) / kBM;
      int incl = c;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
      }
      for (int i = 0; i < c; ++i) {
        tiles[2 * (carry + incl - c + i)] = e;
        tiles[2 * (carry + incl - c + i) + 1] = i * kBM;
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

// ------------------------------------------------------------- gate/up ----
__global__ __launch_bounds__(kThreads) void k_gateup(
    const uint16_t *__restrict__ x16, const int32_t *__restrict__ x_exp,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ sorted_pairs, int top_k,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ ntiles, Nvfp4 gate, Nvfp4 up,
    int H, int I, uint16_t *__restrict__ a_out, uint32_t *__restrict__ a_max) {
  const int tile = blockIdx.y;
  if (tile >= ntiles[0]) return;
  const int e = tiles[2 * tile], m0 = tiles[2 * tile + 1];
  const int row0 = offsets[e] + m0;                       // first sorted row of the tile
  const int mrows = min(kBM, offsets[e + 1] - row0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kCols + wave * 16;

  const size_t wrow = (size_t)e * I + n0 + r;
  const uint8_t *pg = gate.packed + wrow * (H / 2);
  const uint8_t *pu = up.packed + wrow * (H / 2);
  const uint8_t *sg = gate.scales + wrow * (H / 16);
  const uint8_t *su = up.scales + wrow * (H / 16);
  const bool a_ok = r < mrows;
  const uint16_t *pa = x16 + (size_t)(a_ok ? sorted_pairs[row0 + r] / top_k : 0) * H;

  f32x4 accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
  for (int kk = 0; kk < H; kk += 128) {
    // H % 32 == 0: a lane's 32 K indices are all inside or all outside; lanes
    // outside feed zeros (the MFMA itself always runs wave-wide)
    const int k = kk + 32 * g;
    const bool k_ok = k < H;
    u32x4 wg = {0, 0, 0, 0}, wu = {0, 0, 0, 0};
    uint32_t cg = 0, cu = 0;
    if (k_ok) {
      wg = *(const u32x4 *)(pg + k / 2);
      wu = *(const u32x4 *)(pu + k / 2);
      cg = *(const uint16_t *)(sg + k / 16);
      cu = *(const uint16_t *)(su + k / 16);
    }
    f16x8 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0, 0, 0, 0};
      if (a_ok && k_ok) v = *(const u32x4 *)(pa + k + 8 * j);
      a[j] = __builtin_bit_cast(f16x8, v);
    }
    const BlockScale bg0 = decode_block_scale(cg & 0xFF), bg1 = decode_block_scale(cg >> 8);
    const BlockScale bu0 = decode_block_scale(cu & 0xFF), bu1 = decode_block_scale(cu >> 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      accg = mfma16x16x32(a[j], dequant8(wg[j], j < 2 ? bg0 : bg1), accg);
      accu = mfma16x16x32(a[j], dequant8(wu[j], j < 2 ? bu0 : bu1), accu);
    }
  }
  // epilogue: lane holds rows 4g+j, column n0 + r
  const float gg = gate.global[e], gu = up.global[e];
  float rmax[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 4 * g + j;
    rmax[j] = 0.0f;
    if (m < mrows) {
      const int tok = sorted_pairs[row0 + m] / top_k;
      const float f = __builtin_ldexpf(1.0f, x_exp[tok] - 14);
      const float G = accg[j] * (gg * f), U = accu[j] * (gu * f);
      const uint16_t ab = f32_to_bf16(gelu_tanh(G) * U);
      a_out[(size_t)(row0 + m) * I + n0 + r] = ab;
      rmax[j] = fabsf(bf16_to_f32(ab));
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) rmax[j] = fmaxf(rmax[j], __shfl_xor(rmax[j], o, kWave));
    const int m = 4 * g + j;
    if (r == 0 && m < mrows) atomicMax(&a_max[row0 + m], __float_as_uint(rmax[j]));
  }
}

// ---------------------------------------------------------------- down ----
constexpr int kMaxI = 2048;  // largest expert intermediate size held in LDS

__global__ __launch_bounds__(kThreads) void k_down(
    const uint16_t *__restrict__ a_in, const uint32_t *__restrict__ a_max,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, Nvfp4 down, int I, int H, uint16_t *__restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_a[];  // [kBM][I + 8] f16
  const int tile = blockIdx.y;
  if (tile >= ntiles[0]) return;
  const int e = tiles[2 * tile], m0 = tiles[2 * tile + 1];
  const int row0 = offsets[e] + m0;
  const int mrows = min(kBM, offsets[e + 1] - row0);
  const int ld = I + 8;
  const int tid = threadIdx.x;
  // stage A rows as f16, each row scaled by 2^(14 - exponent of its max)
  for (int i = tid; i < kBM * (I / 8); i += kThreads) {
    const int m = i / (I / 8), c = (i % (I / 8)) * 8;
    u32x4 o = {0, 0, 0, 0};
    if (m < mrows) {
      const float f = __builtin_ldexpf(1.0f, 14 - row_exponent(__uint_as_float(a_max[row0 + m])));
      const u32x4 v = *(const u32x4 *)(a_in + (size_t)(row0 + m) * I + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16 lo = (f16)(__uint_as_float(v[q] << 16) * f);
        const f16 hi = (f16)(__uint_as_float(v[q] & 0xFFFF0000u) * f);
        o[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
    }
    *(u32x4 *)(s_a + m * ld + c) = o;
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kCols + wave * 16;
  const size_t wrow = (size_t)e * H + n0 + r;
  const uint8_t *pd = down.packed + wrow * (I / 2);
  const uint8_t *sd = down.scales + wrow * (I / 16);
  f32x4 acc = {0, 0, 0, 0};
  for (int kk = 0; kk < I; kk += 128) {
    // I % 32 == 0: a lane's 32 K indices are all inside or all outside; lanes
    // outside feed zeros (the MFMA itself always runs wave-wide)
    const int k = kk + 32 * g;
    const bool k_ok = k < I;
    u32x4 wd = {0, 0, 0, 0};
    uint32_t cd = 0;
    if (k_ok) {
      wd = *(const u32x4 *)(pd + k / 2);
      cd = *(const uint16_t *)(sd + k / 16);
    }
    const BlockScale b0 = decode_block_scale(cd & 0xFF), b1 = decode_block_scale(cd >> 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = {0, 0, 0, 0};
      if (k_ok) v = *(const u32x4 *)(s_a + r * ld + k + 8 * j);
      acc = mfma16x16x32(__builtin_bit_cast(f16x8, v), dequant8(wd[j], j < 2 ? b0 : b1), acc);
    }
  }
  const float gd = down.global[e];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 4 * g + j;
    if (m < mrows) {
      const float f = __builtin_ldexpf(1.0f, row_exponent(__uint_as_float(a_max[row0 + m])) - 14);
      y[(size_t)(row0 + m) * H + n0 + r] = f32_to_bf16(acc[j] * (gd * f));
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
  if (H % kCols || I % kCols || I > kMaxI || E > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOPK)
    return MOE_ERR_UNSUPPORTED;
  if ((long long)T * top_k > 0x7FFFFFFFLL / 2) return MOE_ERR_SHAPE;
  if (ws_bytes < ws_layout(T, top_k, E, H, I).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

bool tensor_null(const nvfp4_tensor *t) { return !t || !t->packed || !t->scales || !t->global; }

}  // namespace

extern "C" int nvfp4_expert_prep(const uint16_t *x_expert, const int32_t *expert_offsets,
                                 int32_t T, int32_t top_k, int32_t E, int32_t H, int32_t I,
                                 void *workspace, size_t ws_bytes, void *stream) {
  if (!expert_offsets || (T > 0 && !x_expert)) return MOE_ERR_NULL;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  MOE_LAUNCH(k_prep, dim3((T + 3) / 4 + 1), dim3(kThreads), 0, (hipStream_t)stream,
                     x_expert, T, H, expert_offsets, E, T * top_k, w.x16, w.x_exp, w.tiles,
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
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  Nvfp4 g{gate->packed, gate->scales, gate->global};
  Nvfp4 u{up->packed, up->scales, up->global};
  MOE_LAUNCH(k_gateup, dim3(I / kCols, w.L.max_tiles), dim3(kThreads), 0,
                     (hipStream_t)stream, w.x16, w.x_exp, expert_offsets, sorted_pairs, top_k,
                     w.tiles, w.ntiles, g, u, H, I, w.a, w.a_max);
  return MOE_OK;
}

extern "C" int nvfp4_expert_down(const nvfp4_tensor *down, const int32_t *expert_offsets,
                                 int32_t T, int32_t top_k, int32_t H, int32_t I,
                                 uint16_t *y_sorted, void *workspace, size_t ws_bytes,
                                 void *stream) {
  if (tensor_null(down) || !expert_offsets || (T > 0 && !y_sorted)) return MOE_ERR_NULL;
  const int E = down->E;
  if (!tensor_ok(down, E, H, I)) return MOE_ERR_SHAPE;
  int st = check_common(T, top_k, E, H, I, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const Ws w = ws_ptrs(workspace, ws_layout(T, top_k, E, H, I));
  Nvfp4 d{down->packed, down->scales, down->global};
  const size_t lds = (size_t)kBM * (I + 8) * 2;
  MOE_LAUNCH(k_down, dim3(H / kCols, w.L.max_tiles), dim3(kThreads), lds,
                     (hipStream_t)stream, w.a, w.a_max, expert_offsets, w.tiles, w.ntiles, d, I,
                     H, y_sorted);
  return MOE_OK;
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
