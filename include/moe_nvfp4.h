/*
 * moe_nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 weight-only MoE expert block.
 *
 * The block is the sparse branch of a Gemma-4-26B-A4B decoder layer
 * ("Gemma 4 26B-A4B (MoE) - Core AI", Architecture: block pseudocode and the
 * router description): route the raw residual to 8 of 128 experts, run each
 * routed token through its expert's GELU-tanh gated MLP (gate and up
 * 2816 -> 704, down 704 -> 2816), and sum the expert outputs with the routing
 * weights.  Expert weights are NVFP4: E2M1 elements in groups of 16 along the
 * input dimension, one E4M3 scale per group, one FP32 scale per tensor
 * ("Gemma-4-26B-A4B-NVFP4-mlx", Quantization recipe; "gemma-4-26B-A4B -
 * NVFP4A16", Quantization details); activations are bf16 (W4A16).
 *
 * The hot path is four calls, in this order, on one stream:
 *     moe_route -> moe_bucket -> nvfp4_expert_mlp -> moe_combine
 * (moe_route_bucket may replace the first two; moe_route_bucket_prep the
 * first two and the expert MLP's prep stage).
 *
 * Conventions for every entry point
 *   - Every pointer is a device pointer owned by the caller (for example
 *     torch.Tensor.data_ptr()).  The library never allocates or frees device
 *     memory and keeps no state between calls; calls are reentrant.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is queued
 *     asynchronously in stream order; no call synchronises the host, copies
 *     memory or calls hipMemset, so the sequence can be captured in a graph.
 *   - bf16 and f16 values are passed as their uint16_t bit patterns.
 *   - Host-detectable errors return a negative status and queue no work; no
 *     call prints, aborts or exits.  NaN/Inf inputs propagate; they are not
 *     validated.
 *   - Integer outputs that the hot path produces are deterministic: the same
 *     inputs give the same bytes on every run (no float atomics anywhere).
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL                */
#define MOE_ERR_SHAPE (-2)       /* a size is out of range or inconsistent    */
#define MOE_ERR_WORKSPACE (-3)   /* workspace NULL or smaller than required   */
#define MOE_ERR_UNSUPPORTED (-4) /* valid shape this library does not handle  */
#define MOE_ERR_LAUNCH (-5)      /* a kernel launch failed (hipGetLastError)  */

/* Limits of this library. */
#define MOE_MAX_EXPERTS 256 /* E                                   */
#define MOE_MAX_TOPK 16     /* top_k                               */

/* Byte layouts of an nvfp4_tensor. */
#define MOE_LAYOUT_CANONICAL 0 /* the row-major layout below (the pages' packed-U8 form) */
#define MOE_LAYOUT_TILED 1     /* the same bytes permuted into 16-row x 128-K tiles      */

/* Weight formats of an nvfp4_tensor (the `format` field). */
#define MOE_FORMAT_NVFP4 0 /* E2M1 x E4M3 per 16 x FP32 per tensor                     */
#define MOE_FORMAT_Q4_0 1  /* (q - 8) * d, fp16 d per 32 ("Gemma 4 26B-A4B (MoE) -
                              Core AI", Compression recipe: the q4_0 grid)           */
#define MOE_FORMAT_AFF4 2  /* q * s + b, fp16 s and b per 32 (same page: aff4)         */

/*
 * One stack of NVFP4 weights, one tensor per expert, canonical layout:
 *   packed [E][N][K/2]  uint8: element k of row n is nibble (k & 1) of byte
 *                       k/2 (low nibble = even k); nibble = E2M1 code,
 *                       bit 3 sign, bits 0..2 index {0,.5,1,1.5,2,3,4,6}.
 *   scales [E][N][K/16] uint8: OCP E4M3 (fn) code of the block scale of
 *                       elements 16b..16b+15 of row n.
 *   global [E]          float: per-tensor FP32 scale of expert e.
 * Element value: E2M1(code) * E4M3(scale) * global[e].
 * N is the output dimension, K the input ("inner") dimension, K % 32 == 0.
 * Block scales must be finite and non-negative (the quantiser writes no others).
 *
 * MOE_LAYOUT_TILED (what the expert kernels read; made by nvfp4_repack):
 * the same bytes, permuted so that one wave-wide 16-byte load per lane reads
 * one contiguous kilobyte already in matrix-core operand order.  Per expert,
 * rows are grouped in tiles of 16 (N % 16 == 0) and K in units of 128; the
 * units of row tile t are stored one after the other from byte t*16*(K/2).
 * Unit u of tile t holds, for lane l = 16*g + r (g = 0..3, r = 0..15), the 16
 * canonical bytes of row 16t+r covering k = 128u + 32g .. 128u + 32g + 31 at
 * byte 1024u + 16l (a last, partial unit holds only the lanes with k < K).
 * Scales likewise: tile t starts at byte t*K, unit u at +128u, lane l at +2l
 * holds the two scale bytes of row 16t+r for k = 128u + 32g .. +31.
 * Sizes per expert are unchanged: N*K/2 and N*K/16 bytes.
 *
 * The int4 formats (MOE_FORMAT_Q4_0, MOE_FORMAT_AFF4) use the same struct:
 *   packed [E][N][K/2]  uint8: unsigned codes q = 0..15, nibble order as above.
 *   scales  Q4_0: [E][N][K/32] fp16 d;  AFF4: [E][N][K/32][2] fp16 (s, b),
 *                       for elements 32b..32b+31 of row n.
 *   global  not read (may be NULL).
 * Element value: Q4_0 (q - 8) * d, AFF4 q * s + b.  The expert kernels
 * multiply each weight rounded once to f16 (round to nearest even; a zero
 * weight may come out as +0 where the exact product is -0).  Scales and
 * biases must be finite, and for Q4_0 |d| <= 8188 (so that 8d is finite).  Tiled
 * int4 stacks use the same tiles, with the 8 nibbles of every packed dword
 * (elements j = 0..7, canonical bits 4j..4j+3) permuted so that byte b holds
 * element b in its low nibble and element b + 4 in its high nibble, and the
 * scales of lane l of unit u of tile t at byte t*K*SB/2 + 64*SB*u + SB*l
 * (SB = 2 for Q4_0, 4 for AFF4).
 */
typedef struct {
  const uint8_t *packed;
  const uint8_t *scales;
  const float *global;
  int32_t E, N, K;
  int32_t layout; /* MOE_LAYOUT_CANONICAL or MOE_LAYOUT_TILED */
  int32_t format; /* MOE_FORMAT_NVFP4, MOE_FORMAT_Q4_0 or MOE_FORMAT_AFF4 */
} nvfp4_tensor;

/*
 * moe_route -- the router ("Gemma 4 26B-A4B (MoE) - Core AI", Architecture,
 * router description): RMSNorm of the raw residual without a learned weight,
 * times the learned per-channel `router_scale` and H^-0.5, linear to E
 * logits, softmax over all E in fp32, top-k, renormalise the k probabilities
 * to sum 1, multiply by per_expert_scale at the chosen ids.
 *
 *   x                [T][H] bf16   raw residual
 *   w_router         [E][H] bf16   router projection
 *   router_scale     [H]    bf16
 *   per_expert_scale [E]    bf16
 *   logit_bias       [E]    float  or NULL; added to the logits (a device to
 *                                  skew expert popularity; zero on the pages)
 *   eps                            RMSNorm epsilon (1e-6), inside the sqrt
 *   topk_idx  out [T][top_k] int32 chosen expert ids, order unspecified;
 *                                  ties on the logit go to the lower id
 *   topk_w    out [T][top_k] float routing weights (renormalised x pes)
 *   topk_w_raw out [T][top_k] float or NULL: renormalised weights before pes
 *   logits    out [T][E] float or NULL: the logits.  With NULL they never
 *                                  leave the chip: one workgroup per 64
 *                                  tokens computes every expert's logit into
 *                                  LDS and selects there (no scratch memory).
 * Arithmetic: the logits accumulate in fp32 with no rounding of the
 * normalised activation (the per-token 1/rms factor is applied to the dot
 * product); softmax and renormalisation in fp32.
 * Errors: MOE_ERR_NULL for a required NULL; MOE_ERR_SHAPE for T < 0, H <= 0,
 * H % 64, E <= 0, top_k <= 0 or top_k > E; MOE_ERR_UNSUPPORTED for
 * E > MOE_MAX_EXPERTS, E % 16 or top_k > MOE_MAX_TOPK.  T == 0 is a no-op.
 */
int moe_route(const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
              const uint16_t *per_expert_scale, const float *logit_bias, int32_t T, int32_t H,
              int32_t E, int32_t top_k, float eps, int32_t *topk_idx, float *topk_w,
              float *topk_w_raw, float *logits, void *stream);

/*
 * moe_bucket -- sort the T*top_k (token, slot) pairs by expert, the
 * sort-by-expert step of a grouped GEMM ("Gemma 4 26B-A4B (MoE) - Core AI",
 * Decode only: the batched sort-by-expert kernel for more than one token).
 * Pair id p = t*top_k + j.  Order is (expert, t, j): a stable counting sort.
 *
 *   topk_idx        [T][top_k] int32  expert ids in [0, E)
 *   expert_offsets  out [E+1] int32   bucket e is sorted_pairs[off[e] .. off[e+1])
 *   sorted_pairs    out [T*top_k] int32 pair ids in sorted order
 *   pair_rank       out [T*top_k] int32 position of pair p in sorted_pairs
 *   workspace       >= moe_bucket_workspace_bytes(T, top_k, E) bytes (the size
 *                   also holds moe_route_bucket's split router sums); its
 *                   first int32 is the device error word: the number of pairs
 *                   whose id was outside [0, E).  Such pairs are placed after
 *                   every bucket (positions >= off[E]), go to no expert and
 *                   get pair_rank -1, so moe_combine adds nothing for them.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (T < 0, top_k <= 0, E <= 0),
 * MOE_ERR_UNSUPPORTED (E > MOE_MAX_EXPERTS, top_k > MOE_MAX_TOPK),
 * MOE_ERR_WORKSPACE.
 */
int moe_bucket(const int32_t *topk_idx, int32_t T, int32_t top_k, int32_t E,
               int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_rank,
               void *workspace, size_t ws_bytes, void *stream);
size_t moe_bucket_workspace_bytes(int32_t T, int32_t top_k, int32_t E);

/*
 * moe_route_bucket -- moe_route followed by moe_bucket in one call, with the
 * same arguments as the two calls.  For decode batches (T <= 64, H <= 4096)
 * the output bytes are those of the two calls (topk_idx, topk_w, topk_w_raw,
 * logits, expert_offsets, sorted_pairs, pair_rank and the workspace error
 * word), and the top-k selection and the bucketing run in one kernel after
 * the logits kernel, which saves a launch on the latency-bound decode path:
 * one wave per token over ceil(T/4) workgroups, the last of which to finish
 * does the bucketing (no workgroup waits for another).  For more tokens the
 * logits are split along the hidden dimension over more workgroups, whose
 * partial sums (in the workspace) the selection kernel adds in a fixed order:
 * deterministic, within moe_route's error bar, but they may differ from
 * moe_route's logits in the last bits, and ids or weights may differ where
 * two logits are that close; the bucketing is moe_bucket's of the ids chosen.
 * logits may be NULL as in moe_route.
 *   workspace  >= moe_bucket_workspace_bytes(T, top_k, E) bytes (as moe_bucket,
 *              plus the split's partial sums: up to 8 * T * E + 8 * T floats);
 *              word 1 is the call's arrival counter (no initial value needed)
 * Errors: those of moe_route and moe_bucket, checked before any work is
 * queued.
 */
int moe_route_bucket(const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
                     const uint16_t *per_expert_scale, const float *logit_bias, int32_t T,
                     int32_t H, int32_t E, int32_t top_k, float eps, int32_t *topk_idx,
                     float *topk_w, float *topk_w_raw, float *logits, int32_t *expert_offsets,
                     int32_t *sorted_pairs, int32_t *pair_rank, void *workspace, size_t ws_bytes,
                     void *stream);

/*
 * moe_route_bucket_prep -- moe_route_bucket followed by the expert MLP's
 * first stage on the same x: nvfp4_expert_prep(x) when norm_weight is NULL,
 * else nvfp4_expert_prep_rmsnorm(x, norm_weight, norm_eps) (the learned norm
 * of the expert input, "Gemma 4 26B-A4B (MoE) - Core AI", Architecture code
 * sketch).  Same arguments as those calls and the same output bytes as
 * moe_route_bucket followed by the prep call, including the expert
 * workspace's f16 rows; queue nvfp4_expert_gate_up and
 * nvfp4_expert_down after it.  For decode batches (moe_route_bucket's
 * one-launch path) the selection kernel's waves also write the expert input,
 * one token row each, beside the bucketing: one launch fewer.
 *   bucket_ws, bucket_ws_bytes   as moe_route_bucket's workspace
 *   norm_weight [H] bf16 or NULL; norm_eps >= 0 (read with norm_weight)
 *   I, expert_ws, expert_ws_bytes   as nvfp4_expert_prep's (I, workspace)
 * Errors: those of moe_route_bucket and of nvfp4_expert_prep(_rmsnorm),
 * checked before any work is queued.
 */
int moe_route_bucket_prep(const uint16_t *x, const uint16_t *w_router,
                          const uint16_t *router_scale, const uint16_t *per_expert_scale,
                          const float *logit_bias, int32_t T, int32_t H, int32_t E, int32_t top_k,
                          float eps, int32_t *topk_idx, float *topk_w, float *topk_w_raw,
                          float *logits, int32_t *expert_offsets, int32_t *sorted_pairs,
                          int32_t *pair_rank, void *bucket_ws, size_t bucket_ws_bytes,
                          const uint16_t *norm_weight, float norm_eps, int32_t I,
                          void *expert_ws, size_t expert_ws_bytes, void *stream);

/*
 * moe_layer_decode -- the whole block for a decode batch in one call: the
 * router, the bucketing, the expert MLP and the weighted combine of
 * moe_route -> moe_bucket -> nvfp4_expert_mlp -> moe_combine, queued as four
 * kernels instead of five, or three up to 32 pairs ("Gemma-4-26B-A4B-IT -
 * UD-Q8KXL (mlx-node)", Performance: decode gains from fusing the per-layer
 * dispatch):
 *   1. the router logits, beside the expert input's f16 rows;
 *   2. the gate/up projection, every workgroup repeating the top-k selection
 *      of every token and the bucketing in LDS (no kernel of their own);
 *   3. the down projection; 4. the combine -- up to 32 pairs one kernel,
 *      each token's pairs in one workgroup that adds them as moe_combine does.
 * Arguments as those calls' (x is also the expert input).  topk_idx, topk_w,
 * topk_w_raw (NULL allowed), expert_offsets, sorted_pairs and pair_rank have
 * the same bytes as the four calls'; so has out above 32 pairs, and up to 32
 * pairs it is within a few bf16 steps of theirs (each expert output computed
 * over the same K in another order of the fp32 sums).
 *   gate, up, down  nvfp4_tensor as nvfp4_expert_mlp's (MOE_LAYOUT_TILED)
 *   out             [T][H] bf16
 *   workspace       >= moe_layer_decode_workspace_bytes(T, top_k, E, H, I)
 *                   bytes; its word at byte moe_layer_decode_error_offset is
 *                   the bucketing's error word (ids outside [0, E))
 * Limits: T <= MOE_DECODE_MAX_TOKENS, T * top_k <= MOE_DECODE_MAX_PAIRS,
 * H <= 4096 (MOE_ERR_UNSUPPORTED beyond); the checks of moe_route and
 * nvfp4_expert_mlp otherwise.  T == 0 queues nothing.
 */
#define MOE_DECODE_MAX_TOKENS 8
#define MOE_DECODE_MAX_PAIRS 64
int moe_layer_decode(const uint16_t *x, const uint16_t *w_router, const uint16_t *router_scale,
                     const uint16_t *per_expert_scale, const float *logit_bias, int32_t T,
                     int32_t H, int32_t E, int32_t top_k, float eps, const nvfp4_tensor *gate,
                     const nvfp4_tensor *up, const nvfp4_tensor *down, int32_t I,
                     int32_t *topk_idx, float *topk_w, float *topk_w_raw,
                     int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *pair_rank,
                     uint16_t *out, void *workspace, size_t ws_bytes, void *stream);
size_t moe_layer_decode_workspace_bytes(int32_t T, int32_t top_k, int32_t E, int32_t H, int32_t I);
size_t moe_layer_decode_error_offset(int32_t T, int32_t top_k, int32_t E);

/*
 * nvfp4_expert_mlp -- every routed (token, expert) pair through its expert:
 * A = gelu_tanh(X Wg^T) * (X Wu^T), Y = A Wd^T ("Gemma 4 26B-A4B (MoE) -
 * Core AI", Architecture: GELU-gated experts in the tanh form; gate/up
 * 2816 -> 704, down 704 -> 2816), with two-level NVFP4 weights
 * (E2M1 x E4M3 block scale x FP32 tensor scale).
 *
 *   x_expert       [T][H] bf16   expert input (the pre-normed residual; may
 *                                alias the router's x)
 *   gate, up       nvfp4_tensor  N = I, K = H, MOE_LAYOUT_TILED
 *   down           nvfp4_tensor  N = H, K = I, MOE_LAYOUT_TILED
 *                  (the expert kernels read the tiled layout only: a stack
 *                  in the canonical layout is rejected and is converted once
 *                  by nvfp4_repack, a pure permutation of its bytes checked
 *                  bit-exact by nvfp4_dequant_bf16.  Repacking per call would
 *                  read and write the whole stack -- 428 MB for a model layer
 *                  -- for every batch.)
 *   expert_offsets [E+1], sorted_pairs [T*top_k]  from moe_bucket
 *   y_sorted       out [T*top_k][H] bf16  expert output of the pair at each
 *                                sorted position (routing weight not applied)
 *   workspace      >= moe_workspace_bytes(T, top_k, E, H, I) bytes
 * Arithmetic: E2M1 x E4M3 products are exact in f16; activations enter the
 * MFMA as f16 after an exact per-row power-of-two rescale (so no bf16 value
 * overflows; values more than 2^29 below the row's largest lose low bits);
 * fp32 accumulation; the FP32 tensor scale and the power of two are applied
 * to the fp32 sums; A is rounded to bf16 between the projections, Y to bf16.
 * The int4 formats (MOE_FORMAT_Q4_0, MOE_FORMAT_AFF4) run on the same kernels
 * with only the weight decode changed: each weight enters the MFMA rounded
 * once to f16 (one fused f16 multiply-add of the code with its block's scale
 * and bias).  gate and up must have the same format; down may differ.
 * Errors: MOE_ERR_NULL; MOE_ERR_SHAPE (T < 0, top_k <= 0, H or I <= 0,
 * descriptor shapes not [E][I][H], [E][I][H], [E][H][I] with one E);
 * MOE_ERR_UNSUPPORTED (H % 64, I % 64, E > MOE_MAX_EXPERTS,
 * top_k > MOE_MAX_TOPK, a descriptor not in MOE_LAYOUT_TILED, an unknown
 * format or gate and up of different formats, one expert's packed tensor or
 * the activation copies past 2 GiB); MOE_ERR_WORKSPACE.
 */
int nvfp4_expert_mlp(const uint16_t *x_expert, const nvfp4_tensor *gate, const nvfp4_tensor *up,
                     const nvfp4_tensor *down, const int32_t *expert_offsets,
                     const int32_t *sorted_pairs, int32_t T, int32_t top_k, int32_t H, int32_t I,
                     uint16_t *y_sorted, void *workspace, size_t ws_bytes, void *stream);
size_t moe_workspace_bytes(int32_t T, int32_t top_k, int32_t E, int32_t H, int32_t I);

/*
 * nvfp4_expert_mlp_noalloc -- nvfp4_expert_mlp for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the
 * workspace, the same output bytes.  The workspace is a file-scope device
 * array of MOE_NOALLOC_MAX_WORKSPACE_BYTES inside the library, one per GPU,
 * held until the process ends; the call allocates nothing (no hipMalloc, no
 * allocating library routine).  Every call on a GPU shares that GPU's array
 * and leaves its last contents there, so calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race.
 * Errors: those of nvfp4_expert_mlp; MOE_ERR_WORKSPACE when
 * moe_workspace_bytes(T, top_k, E, H, I) exceeds
 * MOE_NOALLOC_MAX_WORKSPACE_BYTES (at the model's H = 2816, I = 704,
 * top_k = 8: up to 495 tokens); MOE_ERR_LAUNCH when the array's device
 * address cannot be looked up.
 */
#define MOE_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)8 << 20)
int nvfp4_expert_mlp_noalloc(const uint16_t *x_expert, const nvfp4_tensor *gate,
                             const nvfp4_tensor *up, const nvfp4_tensor *down,
                             const int32_t *expert_offsets, const int32_t *sorted_pairs, int32_t T,
                             int32_t top_k, int32_t H, int32_t I, uint16_t *y_sorted,
                             void *stream);

/*
 * The three stages of nvfp4_expert_mlp as separate calls, for callers that
 * want to time or overlap them; queued in this order with the same workspace
 * they give the same bytes as nvfp4_expert_mlp.
 *   nvfp4_expert_prep:    per-token power-of-two rescale of x_expert to f16
 *                         ([T][H] in the workspace), and clears the per-row
 *                         max of A.  It does not read the
 *                         routing, so it may run concurrently with moe_route
 *                         and moe_bucket (on another stream or graph branch),
 *                         as long as it completes before nvfp4_expert_gate_up.
 *   nvfp4_expert_gate_up: A = gelu_tanh(X Wg^T) * (X Wu^T) for every sorted
 *                         row, bf16, kept in the workspace.
 *   nvfp4_expert_down:    y_sorted = A Wd^T.
 * Arguments, layouts and errors as for nvfp4_expert_mlp.  The workspace
 * layout depends on (T, top_k, E, H, I) only, so all three calls must be given
 * the same values.
 */
int nvfp4_expert_prep(const uint16_t *x_expert, int32_t T, int32_t top_k, int32_t E, int32_t H,
                      int32_t I, void *workspace, size_t ws_bytes, void *stream);
int nvfp4_expert_gate_up(const nvfp4_tensor *gate, const nvfp4_tensor *up,
                         const int32_t *expert_offsets, const int32_t *sorted_pairs, int32_t T,
                         int32_t top_k, int32_t H, int32_t I, void *workspace, size_t ws_bytes,
                         void *stream);
int nvfp4_expert_down(const nvfp4_tensor *down, const int32_t *expert_offsets, int32_t T,
                      int32_t top_k, int32_t H, int32_t I, uint16_t *y_sorted, void *workspace,
                      size_t ws_bytes, void *stream);

/*
 * moe_combine -- the weighted sum over a token's routed experts
 * ("Gemma 4 26B-A4B (MoE) - Core AI", Architecture: sum over k of w_k h2_k):
 *   out[t] = sum_{j=0..top_k-1} topk_w[t][j] * y_sorted[pair_rank[t*top_k+j]]
 * summed in the fixed order j = 0, 1, ... in fp32, rounded once to bf16.
 *   y_sorted [T*top_k][H] bf16, topk_w [T][top_k] float, pair_rank [T*top_k]
 *   out      out [T][H] bf16
 * A pair whose rank is outside [0, T*top_k) contributes nothing.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (T < 0, top_k <= 0, H <= 0, H % 8),
 * MOE_ERR_UNSUPPORTED (top_k > MOE_MAX_TOPK).
 */
int moe_combine(const uint16_t *y_sorted, const float *topk_w, const int32_t *pair_rank, int32_t T,
                int32_t top_k, int32_t H, uint16_t *out, void *stream);

/*
 * The learned norms of the layer ("Gemma 4 26B-A4B (MoE) - Core AI",
 * Architecture code sketch):
 *     h2 = experts(pre_feedforward_layernorm_2(residual), idx)
 *     h2 = post_feedforward_layernorm_2(sum_k w_k h2_k)
 *     x  = (residual + post_feedforward_layernorm(h1 + h2)) * layer_scalar
 * where h1 is the output of the layer's dense branch (outside the block).
 * Each norm is an RMSNorm with a multiplicative weight:
 *   rmsnorm(v) = v / sqrt(mean(v^2) + eps) * norm_weight     (fp32)
 * (a checkpoint that stores the weight as an offset from 1 passes 1 + w).
 *
 * nvfp4_expert_prep_rmsnorm -- nvfp4_expert_prep with x_expert =
 * rmsnorm(x): the norm is computed from the bf16 row of x in fp32 and feeds
 * the expert kernels' per-row f16 rescale directly (no bf16 rounding of the
 * normed row).  Queue it in place of nvfp4_expert_prep, before
 * nvfp4_expert_gate_up, with the same workspace and shape arguments.
 *   x            [T][H] bf16 (the raw residual; the router reads the same x)
 *   norm_weight  [H] bf16 (pre_feedforward_layernorm_2)
 * Errors: those of nvfp4_expert_prep; MOE_ERR_NULL (norm_weight);
 * MOE_ERR_SHAPE (eps < 0 or NaN).
 */
int nvfp4_expert_prep_rmsnorm(const uint16_t *x, const uint16_t *norm_weight, float eps, int32_t T,
                              int32_t top_k, int32_t E, int32_t H, int32_t I, void *workspace,
                              size_t ws_bytes, void *stream);

/*
 * moe_combine_rmsnorm -- moe_combine followed by the norms of the layer step:
 *   s  = sum_j topk_w[t][j] * y_sorted[pair_rank[t*top_k+j]]   (fp32, j order)
 *   h2 = rmsnorm(s, post_norm2_weight)                          (fp32)
 *   with post_norm_weight:
 *     out[t] = (residual[t] + rmsnorm(h1[t] + h2, post_norm_weight))
 *              * layer_scalar                                   (one bf16 rounding)
 *   without (NULL): out[t] = h2 (the sparse branch's output, one bf16
 *     rounding; h1 and residual must then be NULL, layer_scalar is unused)
 *   post_norm2_weight  [H] bf16 (post_feedforward_layernorm_2)
 *   h1                 [T][H] bf16 or NULL (zero): the dense branch's output
 *   post_norm_weight   [H] bf16 or NULL (post_feedforward_layernorm)
 *   residual           [T][H] bf16, required with post_norm_weight
 *   out                [T][H] bf16; may be the same buffer as residual or h1
 *                      (each element is read before it is written, by one
 *                      thread)
 * Errors: as moe_combine; MOE_ERR_NULL (post_norm2_weight, or residual with
 * post_norm_weight); MOE_ERR_SHAPE (eps < 0 or NaN; h1 or residual without
 * post_norm_weight); MOE_ERR_UNSUPPORTED (H > 8192).
 */
int moe_combine_rmsnorm(const uint16_t *y_sorted, const float *topk_w, const int32_t *pair_rank,
                        const uint16_t *post_norm2_weight, const uint16_t *h1,
                        const uint16_t *post_norm_weight, const uint16_t *residual, float eps,
                        float layer_scalar, int32_t T, int32_t top_k, int32_t H, uint16_t *out,
                        void *stream);

/*
 * nvfp4_quantize -- weight preparation: the block quantiser of the
 * "Gemma-4-26B-A4B-it-NVFP4" README (S_block = max|w|/6 over 16 contiguous
 * inputs, q = clip(round(w / S_block), -6, 6)) in its two-level form.
 * Per expert tensor W [N][K] (bf16):
 *   g = fl32(max|W| / 2688)   (2688 = 6 * 448: largest E2M1 x largest E4M3)
 *   block scale code = nearest E4M3 (ties to even, saturate at 448) of
 *                      amax_block / (6 g), evaluated in IEEE double
 *   element code     = nearest E2M1 (ties to even) of
 *                      clip(w / (E4M3(code) * g), -6, 6) in double; a block
 *                      scale of 0 gives code 0; a zero magnitude gives code 0.
 *   w       [E][N][K] bf16 in;  K % 32 == 0
 *   out     packed, scales, global as in nvfp4_tensor (non-const pointers)
 * The result is bit-identical run to run.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (E, N <= 0, K <= 0, K % 32).
 */
int nvfp4_quantize(const uint16_t *w, int32_t E, int32_t N, int32_t K, uint8_t *packed,
                   uint8_t *scales, float *global, void *stream);

/*
 * nvfp4_repack -- weight preparation: canonical -> MOE_LAYOUT_TILED (a pure
 * permutation of bytes, and of the nibbles of int4 formats, see
 * nvfp4_tensor), for every format.  src must be canonical; the outputs have
 * src's sizes and must not overlap src.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (E, N <= 0, N % 16, K <= 0, K % 32),
 * MOE_ERR_UNSUPPORTED (src not canonical, unknown format).
 */
int nvfp4_repack(const nvfp4_tensor *src, uint8_t *packed_tiled, uint8_t *scales_tiled,
                 void *stream);

/*
 * nvfp4_dequant_bf16 -- decode expert e of a stack to bf16 without the FP32
 * tensor scale: out[n][k] = E2M1(code[n][k]) * E4M3(scale[n][k/16]), which
 * is exact in bf16 ("Gemma-4-26B-A4B-NVFP4-mlx", Notes: E2M1 x per-16 E4M3
 * block scale x per-tensor F32).  A check of the unpacking used by the
 * expert kernels.
 *   out [N][K] bf16
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (e outside [0, E), N or K <= 0, K % 32),
 * MOE_ERR_UNSUPPORTED (a format other than MOE_FORMAT_NVFP4).
 */
int nvfp4_dequant_bf16(const nvfp4_tensor *w, int32_t e, uint16_t *out, void *stream);

/*
 * moe_dequant_f16 -- the f16 weights the expert kernels multiply, for expert
 * e of a stack of any format and layout, through the kernels' own decode:
 * NVFP4 E2M1 * E4M3 (exact, without the FP32 tensor scale); Q4_0 and AFF4
 * the value rounded once to f16.  A check of the weight decode.
 *   out [N][K] fp16 bit patterns
 * Errors: as nvfp4_dequant_bf16, MOE_ERR_UNSUPPORTED (unknown format).
 */
int moe_dequant_f16(const nvfp4_tensor *w, int32_t e, uint16_t *out, void *stream);

/* Text of a status code (static storage). */
const char *moe_status_str(int status);

/* ABI version of this header: (major << 16) | minor (3.0: moe_combine_rmsnorm takes the
 * layer step's h1 and outer norm; moe_route's logits may be NULL). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */
