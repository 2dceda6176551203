// moe_layer_decode: the whole expert block of a decode batch (T <= 8) in
// four launches instead of five -- the router logits with the expert-input
// prep, the gate/up projection with the top-k selection and the bucketing
// folded in, the down projection, the combine -- or in three, with the down
// projection and the combine in one kernel, up to kDecodeCombineMaxP pairs ("Gemma-4-26B-A4B-IT -
// UD-Q8KXL (mlx-node)", Performance: the per-layer dispatch fused for
// decode).
#include "common.h"

namespace moe {
int launch_route_logits_prep(const uint16_t *x, const uint16_t *w_router,
                             const uint16_t *router_scale, const float *logit_bias, int T, int H,
                             int E, float eps, float *logits, const PrepArgs &pa, hipStream_t s);
int launch_decode_gate_up(const float *logits, const uint16_t *pes, int T, int top_k, int E, int H,
                          int I, const nvfp4_tensor *gate, const nvfp4_tensor *up,
                          int32_t *topk_idx, float *topk_w, float *topk_w_raw, int32_t *offsets,
                          int32_t *sorted, int32_t *rank, int32_t *err, void *expert_ws,
                          hipStream_t s);
int launch_decode_down_combine(const int32_t *topk_idx, const float *topk_w, const int32_t *rank,
                               int T, int top_k, int E, int H, int I, const nvfp4_tensor *down,
                               void *expert_ws, uint16_t *out, hipStream_t s);
// Batches of up to this many pairs take the down projection and the combine
// in one launch: each token's pairs in one workgroup, its expert weights read
// once per token (a batch of few tokens shares few experts); larger batches
// keep the expert-major down GEMV, which reads each expert's weights once.
#ifndef MOE_DECODE_COMBINE_MAX_P
#define MOE_DECODE_COMBINE_MAX_P 32
#endif
constexpr int kDecodeCombineMaxP = MOE_DECODE_COMBINE_MAX_P;
}  // namespace moe

namespace {
// Workspace: the logits [T][E] f32, the error word, the expert outputs
// y_sorted [T * top_k][H] bf16, the expert MLP's workspace.
struct LayerWs {
  size_t err, y, expert, total;
};
LayerWs layer_ws(int T, int top_k, int E, int H, int I) {
  LayerWs L;
  L.err = moe_align_up((size_t)T * E * 4, 256);
  L.y = L.err + 256;
  L.expert = L.y + moe_align_up((size_t)T * top_k * H * 2, 256);
  L.total = L.expert + moe_workspace_bytes(T, top_k, E, H, I);
  return L;
}
bool tensor_null(const nvfp4_tensor *t) {
  return !t || !t->packed || !t->scales || (t->format == MOE_FORMAT_NVFP4 && !t->global);
}
bool format_known(int f) { return f >= MOE_FORMAT_NVFP4 && f <= MOE_FORMAT_AFF4; }
}  // namespace

extern "C" size_t moe_layer_decode_workspace_bytes(int32_t T, int32_t top_k, int32_t E, int32_t H,
                                                   int32_t I) {
  if (T < 0 || top_k <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
  return layer_ws(T, top_k, E, H, I).total;
}

extern "C" size_t moe_layer_decode_error_offset(int32_t T, int32_t top_k, int32_t E) {
  if (T < 0 || top_k <= 0 || E <= 0) return 0;
  return moe_align_up((size_t)T * E * 4, 256);
}

extern "C" int moe_layer_decode(const uint16_t *x, const uint16_t *w_router,
                                const uint16_t *router_scale, const uint16_t *per_expert_scale,
                                const float *logit_bias, int32_t T, int32_t H, int32_t E,
                                int32_t top_k, float eps, const nvfp4_tensor *gate,
                                const nvfp4_tensor *up, const nvfp4_tensor *down, int32_t I,
                                int32_t *topk_idx, float *topk_w, float *topk_w_raw,
                                int32_t *expert_offsets, int32_t *sorted_pairs,
                                int32_t *pair_rank, uint16_t *out, void *workspace,
                                size_t ws_bytes, void *stream) {
  using namespace moe;
  if (!w_router || !router_scale || !per_expert_scale || !expert_offsets || !workspace ||
      tensor_null(gate) || tensor_null(up) || tensor_null(down))
    return MOE_ERR_NULL;
  if (T > 0 && (!x || !topk_idx || !topk_w || !sorted_pairs || !pair_rank || !out))
    return MOE_ERR_NULL;
  if (T < 0 || H <= 0 || H % 64 || I <= 0 || E <= 0 || top_k <= 0 || top_k > E)
    return MOE_ERR_SHAPE;
  if (gate->E != E || gate->N != I || gate->K != H || up->E != E || up->N != I || up->K != H ||
      down->E != E || down->N != H || down->K != I)
    return MOE_ERR_SHAPE;
  if (E > MOE_MAX_EXPERTS || E % 16 || top_k > MOE_MAX_TOPK || I % 64 || H > 4096 ||
      T > MOE_DECODE_MAX_TOKENS || T * top_k > MOE_DECODE_MAX_PAIRS)
    return MOE_ERR_UNSUPPORTED;
  if (gate->layout != MOE_LAYOUT_TILED || up->layout != MOE_LAYOUT_TILED ||
      down->layout != MOE_LAYOUT_TILED || !format_known(gate->format) ||
      gate->format != up->format || !format_known(down->format))
    return MOE_ERR_UNSUPPORTED;
  const LayerWs L = layer_ws(T, top_k, E, H, I);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_OK;
  char *ws = (char *)workspace;
  float *logits = (float *)ws;
  int32_t *err = (int32_t *)(ws + L.err);
  void *expert_ws = ws + L.expert;
  PrepArgs pa{};
  int st = expert_prep_buffers(T, top_k, E, H, I, expert_ws, ws_bytes - L.expert, &pa.x16,
                               &pa.x_exp, &pa.a_max);
  if (st != MOE_OK) return st;
  pa.x = x;
  pa.norm_w = nullptr;
  pa.norm_eps = 0.0f;
  pa.H = H;
  pa.P = T * top_k;
  hipStream_t s = (hipStream_t)stream;
  st = launch_route_logits_prep(x, w_router, router_scale, logit_bias, T, H, E, eps, logits, pa, s);
  if (st != MOE_OK) return st;
  st = launch_decode_gate_up(logits, per_expert_scale, T, top_k, E, H, I, gate, up, topk_idx, topk_w,
                             topk_w_raw, expert_offsets, sorted_pairs, pair_rank, err, expert_ws, s);
  if (st != MOE_OK) return st;
  if (T * top_k <= kDecodeCombineMaxP)
    return launch_decode_down_combine(topk_idx, topk_w, pair_rank, T, top_k, E, H, I, down,
                                      expert_ws, out, s);
  uint16_t *y = (uint16_t *)(ws + L.y);
  st = nvfp4_expert_down(down, expert_offsets, T, top_k, H, I, y, expert_ws, ws_bytes - L.expert,
                         stream);
  if (st != MOE_OK) return st;
  return moe_combine(y, topk_w, pair_rank, T, top_k, H, out, stream);
}
