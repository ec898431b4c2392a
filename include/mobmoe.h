/*
 * libmobmoe -- MobileMoE MoE-FFN layer forward on AMD Instinct MI355X (gfx950).
 *
 * The layer (eq. (*) of "MobileMoE: Scaling On-Device Mixture of Experts",
 * close reading on paper-archivist.com, section "MoE preliminaries and three
 * design factors"):
 *
 *     y = sum_{i in top-k(x)} router_i(x) * FFN_i(x)  +  FFN_s(x)
 *
 * with E routed SwiGLU experts of hidden size h, top-k selection by an FP32
 * router, one always-on shared SwiGLU expert of hidden size h_s, INT4
 * symmetric group-32 weights with FP32 scales (eq. (6), section
 * "Quantisation-aware training") and per-token dynamic INT8 activations.
 * The split into calls follows the custom MoE operator of the section
 * "Custom MoE kernel": top-k selection, count-sort of tokens by expert,
 * one fused gate/up product per expert, SwiGLU, down product, and a weighted
 * scatter back through the inverse permutation.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every call returns an mm_status and never throws or aborts.
 *  - All pointers named "device" point to device memory (hipMalloc or a torch
 *    CUDA tensor); "host" pointers point to host memory.  Device pointers must
 *    be 16-byte aligned (MM_ERR_ALIGN otherwise).
 *  - The caller owns every buffer, including workspace.  The library keeps no
 *    pointer past the call and allocates no device memory.
 *  - Work is queued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream).  No call synchronises or reads device memory back.
 *    Buffers must stay alive until the queued work has finished.
 *  - All argument checks happen on the host before anything is queued; a
 *    rejected call queues nothing.  A HIP launch failure returns MM_ERR_HIP;
 *    mm_last_error_string() then describes it (per host thread).
 *  - T == 0 (no tokens) is a valid no-op returning MM_OK.
 *  - Inputs and outputs must not alias.
 *  - Results are deterministic: identical inputs give identical bits for any
 *    stream.  No floating-point atomics are used.
 *
 * Shape limits of this version: 1 <= E <= 64, 1 <= k <= min(8, E),
 * d_model, hidden and shared_hidden multiples of 64 (shared_hidden may be 0:
 * no shared expert), T*k <= 2^24.
 *
 * "Sorted order" below means expert-contiguous order: position p in
 * [expert_offsets[e], expert_offsets[e+1]) holds one (token, slot) routed to
 * expert e, and perm[p] = token*k + slot.
 */
#ifndef MOBMOE_H
#define MOBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mm_status {
  MM_OK = 0,
  MM_ERR_NULL = 1,       /* a required pointer is NULL                      */
  MM_ERR_SHAPE = 2,      /* a size is out of range or inconsistent          */
  MM_ERR_ALIGN = 3,      /* a device pointer is not 16-byte aligned         */
  MM_ERR_FORMAT = 4,     /* unknown weight format, gating rule or dtype     */
  MM_ERR_WORKSPACE = 5,  /* workspace smaller than mm_workspace_bytes()     */
  MM_ERR_HIP = 6         /* a HIP runtime call or kernel launch failed      */
} mm_status;

/* Weight formats (mm_layer_desc.wfmt). */
enum {
  MM_W_F32 = 0,      /* FP32 weights, FP32 activations, no quantisation         */
  MM_W_INT4G32 = 1,  /* INT4 group-32 weights (prepacked), INT8 activations     */
  MM_W_BF16 = 2      /* BF16 weights and activations, FP32 accumulation         */
};

/* Gating rules (mm_layer_desc.gating): one of the first two, optionally
   with MM_GATE_BIAS_SELECT_ONLY added. */
enum {
  MM_GATE_SOFTMAX = 0,      /* softmax over all E logits, no renormalisation    */
  MM_GATE_SIGMOID_NORM = 1, /* sigmoid of each selected logit, divided by their
                               sum over the k selected (training-time gate of the
                               "Pre-training" section)                           */
  MM_GATE_BIAS_SELECT_ONLY = 2 /* the router bias steers the selection only: the
                               experts are ranked by logit + bias, the gate
                               weights use the logits without it (the load-
                               balancing bias of the "Pre-training" section)     */
};

/* Output dtypes (mm_layer_desc.out_dtype): y of mm_combine. */
enum { MM_OUT_F32 = 0, MM_OUT_BF16 = 1 };

/* Workspace queries (mm_workspace_bytes `which`). */
enum {
  MM_WS_ROUTE = 0,
  MM_WS_GATEUP = 1,
  MM_WS_DOWN = 2,
  MM_WS_SHARED = 3,
  MM_WS_MAX = 4,     /* the largest of the above: one buffer serves every call */
  MM_WS_FORWARD = 5, /* mm_moe_forward: every intermediate of the layer */
  MM_WS_DECODE = 6   /* mm_moe_decode: its state and intermediates (any T <= 4) */
};

typedef struct mm_layer_desc {
  int32_t d_model;        /* d: token width                                   */
  int32_t n_experts;      /* E: routed experts                                */
  int32_t hidden;         /* h: routed expert hidden size                     */
  int32_t shared_hidden;  /* h_s: shared expert hidden size, 0 = none         */
  int32_t top_k;          /* k: experts per token                             */
  int32_t wfmt;           /* MM_W_*                                           */
  int32_t gating;         /* MM_GATE_*                                        */
  int32_t out_dtype;      /* MM_OUT_*                                         */
} mm_layer_desc;

/*
 * A weight tensor.  For MM_W_INT4G32 `data` is the prepacked nibble buffer and
 * `scales` its prepacked FP32 scales, both written by mm_prepack_int4g32().
 * For MM_W_F32 `data` is FP32 row-major and for MM_W_BF16 it is BF16
 * (uint16) row-major; `scales` must then be NULL.  Expert tensors are stacked
 * [E][rows][cols].  Gate/up tensors have 2*h rows: rows 0..h-1 are the gate
 * projection and rows h..2h-1 the up projection.
 */
typedef struct mm_weight {
  const void* data;     /* device */
  const float* scales;  /* device, INT4 only */
} mm_weight;

/* ---------------------------------------------------------------- helpers */

const char* mm_version(void);
const char* mm_status_string(mm_status s);
/* Description of the last failure on the calling host thread ("" if none). */
const char* mm_last_error_string(void);

/* Bytes of caller workspace the named call needs for T tokens (0 if none).
 * Returns 0 for an invalid descriptor.  Workspace holds no state between
 * calls; calls that share a workspace buffer must not overlap in time (same
 * stream, or synchronised). */
size_t mm_workspace_bytes(const mm_layer_desc* desc, int64_t T, int32_t which);

/*
 * Offline weight quantisation, eq. (6) with b = 4 and groups of 32 along the
 * input (column) dimension:  s_g = (2 * max|W_g|) / 15 in FP32 with IEEE
 * division, q = clamp(round_half_even(W / s_g), -8, 7); an all-zero group has
 * s_g = 0 and q = 0.
 *   w       device FP32 [rows][cols], cols % 32 == 0
 *   q       device uint8 [rows][cols/2], canonical nibble layout: column c is
 *           in byte c/2, low nibble for even c, 4-bit two's complement
 *   scales  device FP32 [rows][cols/32]
 */
mm_status mm_quantize_int4g32(int64_t rows, int64_t cols, const float* w, uint8_t* q,
                              float* scales, void* stream);

/* Size in bytes of the prepacked nibble buffer and of the prepacked scale
 * buffer for a [rows][cols] INT4 matrix (rows % 32 == 0, cols % 32 == 0). */
size_t mm_prepacked_bytes(int64_t rows, int64_t cols);
size_t mm_prepacked_scale_bytes(int64_t rows, int64_t cols);

/*
 * Rearranges `n_mat` stacked canonical INT4 matrices [n_mat][rows][cols]
 * (layout of mm_quantize_int4g32) into the kernels' layout.  The prepacked
 * layout is private to this library version: pass it only to the calls below.
 * It keeps each group scale as s / 16 in FP32 (the kernels unpack nibbles as
 * 16 q).  For every group with s >= 2^-122 (max|W| >= 7.5 * 2^-122) that
 * quotient is exact and the products are bit-identical to s * sum; below,
 * s / 16 is subnormal and may round, and that group's term is then exact only
 * to within 2^-149 / (s / 16) relative.
 *   q_canon, s_canon   device, canonical nibbles and scales
 *   q_out, s_out       device, n_mat * mm_prepacked_bytes / _scale_bytes
 */
mm_status mm_prepack_int4g32(int64_t n_mat, int64_t rows, int64_t cols, const uint8_t* q_canon,
                             const float* s_canon, uint8_t* q_out, float* s_out, void* stream);

/* FP32 -> BF16 (round to nearest even) conversion of n values (device). */
mm_status mm_convert_bf16(int64_t n, const float* x, uint16_t* y, void* stream);

/* ------------------------------------------------------- the seven calls */

/*
 * FP32 router, top-k selection and gate weights (the section
 * "Pre-training" keeps the router in FP32; eq. (*) weights each selected
 * expert by router_i(x)).
 *   x          device FP32 [T][d]
 *   w_router   device FP32 [E][d]
 *   bias       device FP32 [E] or NULL; added to every logit before selection
 *   topk_idx   device int32 [T][k]   out: selected experts, best first
 *   topk_w     device FP32 [T][k]    out: gate weights
 * Logit of (t, e): 64 partial sums, partial l accumulating x[t][j]*w[e][j]
 * with fused multiply-adds for j = l, l+64, ... ascending; then a balanced
 * pairwise tree (pairs at distance 1, 2, 4, ..., 32); then + bias[e].  Experts
 * are ranked by (logit descending, index ascending).  MM_GATE_SOFTMAX gives
 * w = exp(l_i - max l) / sum over all E of exp(l_e - max l).  With
 * MM_GATE_BIAS_SELECT_ONLY the ranking uses logit + bias[e] and the gate
 * weights the logits without the bias.
 */
mm_status mm_router_topk(const mm_layer_desc* desc, int64_t T, const float* x,
                         const float* w_router, const float* bias, int32_t* topk_idx,
                         float* topk_w, void* stream);

/*
 * Stable count sort of the T*k (token, slot) assignments by expert id
 * (section "Custom MoE kernel": tokens of one expert become contiguous).
 *   topk_idx        device int32 [T*k]
 *   expert_offsets  device int32 [E+1]  out: start of each expert's run,
 *                                        expert_offsets[E] = T*k
 *   perm            device int32 [T*k]  out: sorted position -> token*k+slot
 *   inv_perm        device int32 [T*k]  out: token*k+slot -> sorted position
 *   ws / ws_bytes   device workspace, mm_workspace_bytes(desc, T, MM_WS_ROUTE)
 * Within one expert's run, entries are in ascending token*k+slot order.
 * Ids outside [0, E) are skipped (not counted, not placed); the outputs are then
 * incomplete, but no memory outside the buffers above is touched.
 */
mm_status mm_route_permute(const mm_layer_desc* desc, int64_t T, const int32_t* topk_idx,
                           int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Per-row dynamic INT8 quantisation (eq. (6) read with b = 8 and one
 * group per row): s = (2 * max|v|) / 255, q = clamp(round_half_even(v / s),
 * -128, 127), FP32 with IEEE division; an all-zero row has s = 0, q = 0.
 *   x      device FP32 [rows][cols]
 *   q      device int8 [rows][cols]    out
 *   scale  device FP32 [rows]          out
 */
mm_status mm_act_quant_i8(int64_t rows, int64_t cols, const float* x, int8_t* q, float* scale,
                          void* stream);

/* Layouts of an INT8 code matrix [rows][cols]. */
enum {
  MM_ACT_ROW_MAJOR = 0,   /* code (r, c) at byte r * cols + c                         */
  MM_ACT_GROUP_MAJOR = 1, /* code (r, c) at byte ((c / 32) * rows + r) * 32 + c % 32:
                             the 32 codes of one row and one quantisation group are
                             contiguous, and so are consecutive rows of one group;
                             needs cols % 128 == 0                                    */
  MM_ACT_F16_PAIRED = 2   /* 16-bit values, row-major [rows][cols] (q holds 2 * rows *
                             cols bytes); inside each aligned block of 8 columns,
                             column c (0..7) sits at slot c / 2 (c even) or 4 + c / 2
                             (c odd) and holds the code as an IEEE half value, divided
                             by 16 for c >= 4 (exact).  What the f16 merged products
                             (mm_expert_gateup_pair_f32, mm_expert_down_pair_f32)
                             read; needs cols % 128 == 0                              */
};

/*
 * mm_act_quant_i8 with the codes written in `layout` (MM_ACT_*); the same
 * codes and scales.  MM_ERR_SHAPE for MM_ACT_GROUP_MAJOR with cols % 128 != 0,
 * MM_ERR_FORMAT for an unknown layout.
 */
mm_status mm_act_quant_i8_layout(int64_t rows, int64_t cols, const float* x, int8_t* q,
                                 float* scale, int32_t layout, void* stream);

/*
 * Routed experts' fused gate/up product with SwiGLU (section "Custom MoE
 * kernel"), for every sorted position p of every expert e:
 *   g = x[t] W_gate[e]^T, u = x[t] W_up[e]^T, a = SiLU(g) * u, t = perm[p]/k.
 * MM_W_INT4G32:  act is x_q (int8 [T][d]) with act_scale (FP32 [T]); each
 *   output is s_x * sum_g s_w[g] * isum_g with exact int32 group sums; the row
 *   a is re-quantised per row like mm_act_quant_i8 into h (int8 [T*k][h],
 *   sorted order) and h_scale (FP32 [T*k]).  With h_scale NULL the FP32 rows
 *   a themselves are written to h (FP32 [T*k][h], sorted order) and ws may
 *   be NULL: for callers that apply their own re-quantisation.
 * MM_W_F32 / MM_W_BF16: act is x (FP32 [T][d]), act_scale and h_scale NULL;
 *   h is FP32 (MM_W_F32) or BF16 (MM_W_BF16) [T*k][h], sorted order.  BF16:
 *   x is rounded to BF16 (nearest even) into ws first, products accumulate
 *   in FP32, a is rounded to BF16.
 *   w_gateup        stacked [E][2h][d] (see mm_weight)
 *   perm, expert_offsets  from mm_route_permute
 *   ws / ws_bytes   mm_workspace_bytes(desc, T, MM_WS_GATEUP): INT4 staging
 *                   of the FP32 rows a, or the BF16 copy of x; 0 bytes (ws may
 *                   be NULL) for MM_W_F32
 */
mm_status mm_expert_gateup_swiglu(const mm_layer_desc* desc, int64_t T, const void* act,
                                  const float* act_scale, const int32_t* perm,
                                  const int32_t* expert_offsets, mm_weight w_gateup, void* h,
                                  float* h_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * The routed experts' and the shared expert's gate/up products with SwiGLU
 * (sections "Custom MoE kernel" and "Divide-and-conquer architecture
 * search", Finding 3) in one launch, INT4 weights only: the arithmetic of
 * mm_expert_gateup_swiglu with h_scale = NULL (FP32 hidden rows,
 * bit-identical).  This form takes the exact group sums from the f16 matrix
 * cores (INT8 and INT4 codes are exact f16 values and every partial sum is an
 * integer below 2^24), so each output needs one FP32 multiply-add per group
 * and no integer-to-float conversion; workgroups of four waves share the
 * activation and weight tiles through LDS.
 *   xq, sx            x_q as MM_ACT_F16_PAIRED codes [T][d] and its FP32
 *                     scales [T] (mm_act_quant_i8_layout)
 *   perm, expert_offsets  from mm_route_permute
 *   w_gateup          routed, stacked [E][2h][d]; ws_gateup shared [2h_s][d]
 *   h_r               out: FP32 [T*k][h], sorted order
 *   h_s               out: FP32 [T][h_s]
 * Needs desc->wfmt == MM_W_INT4G32 (else MM_ERR_FORMAT), shared_hidden > 0,
 * d % 128 == 0 and h, h_s % 64 == 0 (else MM_ERR_SHAPE).
 */
mm_status mm_expert_gateup_pair_f32(const mm_layer_desc* desc, int64_t T, const void* xq,
                                    const float* sx, const int32_t* perm,
                                    const int32_t* expert_offsets, mm_weight w_gateup,
                                    mm_weight ws_gateup, float* h_r, float* h_s, void* stream);

/*
 * The routed experts' and the shared expert's down products in one launch on
 * the f16 matrix cores, as mm_expert_gateup_pair_f32 (the arithmetic of
 * mm_expert_down and mm_shared_expert's down product, bit-identical).
 *   hq_r, hs_r   routed hidden rows as MM_ACT_F16_PAIRED codes [T*k][h]
 *                (sorted order) and their scales [T*k]
 *   hq_s, hs_s   shared hidden rows, MM_ACT_F16_PAIRED [T][h_s], scales [T]
 *   expert_offsets  from mm_route_permute
 *   w_down [E][d][h], ws_down [d][h_s]
 *   f            out: FP32 [T*k][d], sorted order (gate weight not applied)
 *   ys           out: FP32 [T][d]
 * Same requirements as mm_expert_gateup_pair_f32.
 */
mm_status mm_expert_down_pair_f32(const mm_layer_desc* desc, int64_t T, const void* hq_r,
                                  const float* hs_r, const void* hq_s, const float* hs_s,
                                  const int32_t* expert_offsets, mm_weight w_down,
                                  mm_weight ws_down, float* f, float* ys, void* stream);

/*
 * Routed experts' down product: f[p] = h[p] W_down[e]^T for every sorted
 * position p of expert e, FP32 [T*k][d] in sorted order (gate weight not yet
 * applied).  INT4: h int8 with h_scale, exact int32 group sums then FP32
 * scales.  F32 / BF16: h as written by mm_expert_gateup_swiglu, h_scale NULL.
 *   w_down  stacked [E][d][h]
 */
mm_status mm_expert_down(const mm_layer_desc* desc, int64_t T, const void* h,
                         const float* h_scale, const int32_t* expert_offsets, mm_weight w_down,
                         float* f, void* ws, size_t ws_bytes, void* stream);

/*
 * The always-on shared expert (section "Divide-and-conquer architecture
 * search", Finding 3): a dense SwiGLU FFN of hidden h_s on every token with
 * weight 1, using the same activation input and arithmetic as the routed
 * experts: ys [T][d] FP32.  w_gateup [2h_s][d], w_down [d][h_s].
 *   ws / ws_bytes  mm_workspace_bytes(desc, T, MM_WS_SHARED)
 * Returns MM_ERR_SHAPE if desc->shared_hidden == 0.
 */
mm_status mm_shared_expert(const mm_layer_desc* desc, int64_t T, const void* act,
                           const float* act_scale, mm_weight w_gateup, mm_weight w_down,
                           float* ys, void* ws, size_t ws_bytes, void* stream);

/*
 * Weighted combine through the inverse permutation (section "Custom MoE
 * kernel"): y[t][c] = fma-chain over j = 0..k-1 of topk_w[t][j] *
 * f[inv_perm[t*k+j]][c], then + ys[t][c] (ys may be NULL).  No atomics.
 *   y  device [T][d], FP32 (MM_OUT_F32) or BF16 (MM_OUT_BF16)
 */
mm_status mm_combine(const mm_layer_desc* desc, int64_t T, const float* f,
                     const int32_t* inv_perm, const float* topk_w, const float* ys, void* y,
                     void* stream);

/*
 * The whole layer in one call: eq. (*) (section "MoE preliminaries and three
 * design factors"), the seven calls above in order with the same arithmetic
 * and bit-identical results, issued as fewer launches on one stream.  The
 * router pass also quantises x (INT4 weights), and the routed and shared
 * products of each kind share one launch, as do their hidden-row quantisers;
 * from 4096 tokens (matrix-core products, FP32 y, no y_norm) the shared down
 * runs after the routed down and does the weighted combine itself, in the
 * combine's order (no separate combine launch).
 *   x                  device FP32 [T][d]
 *   w_router, bias     as mm_router_topk (bias may be NULL)
 *   w_gateup, w_down   routed experts, as mm_expert_gateup_swiglu / mm_expert_down
 *   ws_gateup, ws_down shared expert; ignored (may be zero) when shared_hidden == 0
 *   topk_idx, topk_w   out: device int32 / FP32 [T][k], as mm_router_topk
 *   y                  out: device [T][d], FP32 or BF16 per desc->out_dtype
 *   y_norm, norm_eps   optional (y_norm NULL: not written): FP32 [T][d]
 *                      RMSNorm(y) = y / sqrt(mean_c y^2 + norm_eps), unit gain, for
 *                      the next layer of a decoder stack (outside eq. (*));
 *                      needs FP32 y and norm_eps > 0
 *   ws / ws_bytes      mm_workspace_bytes(desc, T, MM_WS_FORWARD): the routing
 *                      tables, quantised rows and expert outputs of the call
 * Errors as the individual calls; nothing is queued when a check fails.
 */
mm_status mm_moe_forward(const mm_layer_desc* desc, int64_t T, const float* x,
                         const float* w_router, const float* bias, mm_weight w_gateup,
                         mm_weight w_down, mm_weight ws_gateup, mm_weight ws_down,
                         int32_t* topk_idx, float* topk_w, void* y, float* y_norm,
                         float norm_eps, void* ws, size_t ws_bytes, void* stream);

/*
 * mm_moe_forward for a decode step of 1 to 4 tokens as ONE kernel launch
 * (section "Runtime latency": a few tokens are bound by the selected experts'
 * weight bytes, so the separate launches' dependency gaps dominate; section
 * "Custom MoE kernel", principle (2): the layer's steps fused).  Arguments,
 * outputs and errors as mm_moe_forward, with the same arithmetic in the same
 * order, so the results are bit-identical to it.  INT4 weights only
 * (MM_ERR_FORMAT otherwise).  The launch's workgroups pass the routing,
 * hidden rows and expert outputs to one another through `ws`, which holds a
 * small state between calls:
 *   ws / ws_bytes  mm_workspace_bytes(desc, T, MM_WS_DECODE), one size for
 *                  every T <= 4.  Zero-fill it once before its first use;
 *                  every call leaves it ready for the next.  Calls that
 *                  share a ws must not overlap in time (same stream, or
 *                  synchronised).  The uint32 at byte offset 16 counts waits
 *                  inside the kernel that gave up (a call that raises it has
 *                  undefined outputs); only the caller clears it.
 * MM_ERR_SHAPE when mm_moe_decode_supported(desc, T) is 0; MM_ERR_HIP also
 * when the device cannot hold every workgroup of the launch at once (the
 * workgroups wait for one another).
 */
mm_status mm_moe_decode(const mm_layer_desc* desc, int64_t T, const float* x,
                        const float* w_router, const float* bias, mm_weight w_gateup,
                        mm_weight w_down, mm_weight ws_gateup, mm_weight ws_down,
                        int32_t* topk_idx, float* topk_w, void* y, float* y_norm,
                        float norm_eps, void* ws, size_t ws_bytes, void* stream);

/*
 * mm_moe_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without ws / ws_bytes, the same checks and bit-identical
 * results.  Its state and intermediates live in a fixed device array of
 * 512 KiB inside the library, one per GPU, held until the process ends; the
 * call allocates nothing.  The first call on a GPU looks the array up and
 * queues one small kernel on `stream` that clears its state block; every call
 * leaves it cleared.  All calls on one GPU share that array: calls that
 * overlap in time on one GPU (other streams, other threads) race and give
 * undefined results.  MM_ERR_WORKSPACE when the layer needs more than the
 * array holds (4 tokens' rows: 4*k*(h + d) + 4*(h_s + d) floats plus about
 * 21 KB of state, each part rounded up to 256 bytes).
 */
mm_status mm_moe_decode_noalloc(const mm_layer_desc* desc, int64_t T, const float* x,
                                const float* w_router, const float* bias, mm_weight w_gateup,
                                mm_weight w_down, mm_weight ws_gateup, mm_weight ws_down,
                                int32_t* topk_idx, float* topk_w, void* y, float* y_norm,
                                float norm_eps, void* stream);

/* 1 if mm_moe_decode has a form for this layer and T (INT4 weights,
 * 1 <= T <= 4, d % 128 == 0 and d <= 1280, h and h_s (or h_s = 0) multiples
 * of 128 up to 2560, and the weight-streaming products' limits), else 0. */
int32_t mm_moe_decode_supported(const mm_layer_desc* desc, int64_t T);

/*
 * Measurement hook for benchmarks and profilers (not part of eq. (*)): with
 * start and stop both non-NULL (hipEvent_t handles the caller created),
 * every following mm_moe_forward records `start` on its stream right before
 * the launch(es) of its gate/up product stage (the layer's largest product:
 * routed and shared gate/up with SwiGLU, one merged launch where the layer
 * uses one) and `stop` right after them, so the caller can time that stage
 * inside the step with hipEventElapsedTime.  Both NULL switch it off.  The
 * setting is process-wide; set it from one thread while no mm_moe_forward
 * call is in flight.  Returns MM_ERR_NULL if exactly one is NULL.
 */
mm_status mm_set_profile_events(void* start, void* stop);

/* --------------------------------------------------- around the layer */

/*
 * W4A8 dense linear: eq. (6) INT4 group-32 weights with FP32 scales against
 * per-row INT8 activations (section "Quantisation-aware training": every
 * linear layer runs this way, the attention and embedding projections around
 * the MoE-FFN included):
 *   y[r][o] = s_x[r] * (fma chain over g ascending of s_w[o][g] * isum_g(r, o)),
 *   isum_g the exact int32 sum over the 32 inputs of group g; FP32 output.
 *   rows          activation rows (0: no-op)
 *   in_features   K, a positive multiple of 64
 *   out_features  N, a positive multiple of 64; rows * max(K, N) < 2^31
 *   xq, sx        device int8 [rows][K] row-major codes and FP32 [rows] scales
 *                 (mm_act_quant_i8)
 *   w             prepacked INT4 [N][K] (mm_prepack_int4g32 with n_mat = 1) and
 *                 its prepacked scales
 *   y             device FP32 [rows][N]
 * Results are those of the expert down product (same kernels), bit for bit.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN (pointers, 16-byte aligned), MM_ERR_SHAPE.
 */
mm_status mm_linear_w4a8(int64_t rows, int64_t in_features, int64_t out_features,
                         const int8_t* xq, const float* sx, mm_weight w, float* y, void* stream);

/* --------------------------------------------- GQA decode attention, INT8 KV */

/*
 * Grouped-query attention around the MoE-FFN (section "MoE preliminaries and
 * three design factors": each layer is GQA attention plus the FFN; eq. (5):
 * the KV cache is held in b_kv = 8 bits; n_kv = 4, d_h = 64 in "Pre-training").
 * Cache layout, caller-owned: codes [B][n_kv][max_T][d_h] int8 and scales
 * [B][n_kv][max_T] FP32, one symmetric INT8 scale per (position, head) vector
 * by the activation rule (s = 2 max|v| / 255, codes clamp(rint(v / s))).
 * v1 limits: d_h = 64; n_h a multiple of n_kv with n_h / n_kv <= 8.
 */

/* Bytes of one INT8 KV cache (keys or values) of the layout above for B
 * sequences of max_T positions: which = MM_KV_CODES gives the codes
 * (B * n_kv * max_T * d_h, one byte per value: eq. (5)'s b_kv = 8 term for
 * one layer's keys or values), MM_KV_SCALES their FP32 scales (4 bytes per
 * (position, head) vector).  0 for invalid sizes. */
enum { MM_KV_CODES = 0, MM_KV_SCALES = 1 };
size_t mm_kv_cache_bytes(int64_t B, int32_t n_kv, int32_t d_h, int64_t max_T, int32_t which);

/* Workspace of mm_attn_decode_i8 for B sequences of at most max_len positions
 * (0 for invalid sizes). */
size_t mm_attn_workspace_bytes(int64_t B, int32_t n_kv, int64_t max_len);

/*
 * Appends one token's keys and values: k_new, v_new FP32 [B][n_kv][d_h] are
 * quantised per (sequence, head) vector into position pos[b] (device int32
 * [B]) of the caches; positions outside [0, max_T) are skipped.  Codes and
 * scales are bit-identical to mm_act_quant_i8 on the [B * n_kv][d_h] rows.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE.  B = 0 is a no-op.
 */
mm_status mm_kv_append_i8(int64_t B, int32_t n_kv, int32_t d_h, int64_t max_T, const int32_t* pos,
                          const float* k_new, const float* v_new, int8_t* k_cache,
                          int8_t* v_cache, float* k_scale, float* v_scale, void* stream);

/*
 * One new token per sequence: for query head h (key/value head h / (n_h /
 * n_kv)), out[b][h] = sum over t < lens[b] of p_t * s_v[t] v_q[t], p the
 * softmax over t of s_k[t] (q[b][h] . k_q[t]) / sqrt(d_h).  FP32 arithmetic
 * in any order (tolerance-checked against the oracle's double evaluation).
 *   q       device FP32 [B][n_h][d_h] (positions already encoded)
 *   lens    device int32 [B], each in [1, max_len] (clamped to it; a length of
 *           0 gives a zero output row)
 *   max_len host bound on lens, 1 <= max_len <= max_T; sizes the workspace
 *   out     device FP32 [B][n_h][d_h]
 *   ws      device workspace of mm_attn_workspace_bytes(B, n_kv, max_len)
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE, MM_ERR_WORKSPACE.
 */
mm_status mm_attn_decode_i8(int64_t B, int32_t n_h, int32_t n_kv, int32_t d_h, int64_t max_T,
                            int64_t max_len, const int32_t* lens, const float* q,
                            const int8_t* k_cache, const int8_t* v_cache, const float* k_scale,
                            const float* v_scale, float* out, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------
 * Training side of the layer (MobileMoE close reading, section "Pre-training":
 * the MoE stability list balances load through an expert bias updated from
 * the batch, without an auxiliary loss; the efficiency list gives every expert
 * a fixed token buffer, drop-and-pad with capacity factor 1.5; section
 * "Quantisation-aware training": eq. (6) applied as fake quantisation).
 * ------------------------------------------------------------------------- */

/*
 * Aux-loss-free balancing step.  load_e = number of the T*k ids in topk_idx
 * (device int32 [T][k]) equal to e; every bias (device FP32 [E], updated in
 * place) moves by lambda towards balance: + lambda if load_e < T*k/E,
 * - lambda if above, unchanged if equal (compared exactly in integers; one
 * FP32 add).  load (device int32 [E], may be NULL) receives load_e.  Ids
 * outside [0, E) are not counted.  Bit-identical to the oracle.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE (E outside [1, 4096],
 * T*k >= 2^31).  T = 0 is a no-op.
 */
mm_status mm_bias_update(int64_t T, int32_t E, int32_t k, const int32_t* topk_idx, float lambda,
                         float* bias, int32_t* load, void* stream);

/* Per-expert buffer rows of drop-and-pad: ceil((num / den) * T * k / E) in
 * exact integer arithmetic (num / den = 3 / 2 for the factor 1.5); -1 for
 * invalid arguments. */
int64_t mm_drop_pad_capacity(int64_t T, int32_t k, int32_t E, int32_t num, int32_t den);

/*
 * Drop-and-pad dispatch from the stable count sort of mm_route_permute
 * (offsets [E+1], perm and inv_perm [T*k], all device int32) and the ids
 * topk_idx [T][k]: assignments are admitted in token order and the first
 * `capacity` of each expert kept.  Outputs (device int32):
 *   buf       [E][capacity]  assignment id t*k+j of expert e's p-th kept
 *                            assignment, -1 for padding rows
 *   offsets_c [E+1]          exclusive prefix sum of min(load_e, capacity)
 *   perm_c    [T*k]          kept assignments expert by expert, -1 past
 *                            offsets_c[E]
 *   inv_c     [T*k]          row of each assignment in perm_c, -1 if dropped
 * (offsets_c, perm_c, inv_c have the layout of the dropless routing; the
 * combine takes inv_c as its inverse permutation and skips the -1 rows).
 * Bit-identical to the oracle.  buf may be NULL when E * capacity = 0.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE (E outside [1, 4096],
 * negative capacity, E * capacity or T*k >= 2^31).
 */
mm_status mm_drop_pad(int64_t T, int32_t E, int32_t k, int64_t capacity, const int32_t* topk_idx,
                      const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm,
                      int32_t* buf, int32_t* offsets_c, int32_t* perm_c, int32_t* inv_c,
                      void* stream);

/*
 * Fake quantisation of QAT, eq. (6) with b = bits over groups of `group`
 * consecutive elements of each row of x (device FP32 [rows][cols]):
 * s = (2 max|x_g|) / (2^b - 1), u = round_half_even(x / s) (IEEE quotient),
 *   x_bar = s * clamp(u, -2^(b-1), 2^(b-1) - 1)                (FP32)
 * and its straight-through backward (rounding's derivative taken as 1, the
 * clamp's at u):  grad_in = grad_out where u lies in the clamp range, else 0;
 * an all-zero group gives x_bar = 0 and passes the gradient.  x_bar (may be
 * NULL) and the pair grad_out / grad_in (both NULL or both set) are device
 * FP32 [rows][cols]; either or both are computed in one pass.
 * bits 4 or 8; group 32 (cols a multiple of 32) or group = cols (one group
 * per row, cols a multiple of 4).  Bit-identical to the oracle.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE.
 */
mm_status mm_fake_quant(int64_t rows, int64_t cols, int32_t bits, int64_t group, const float* x,
                        float* x_bar, const float* grad_out, float* grad_in, void* stream);

/*
 * Row gather for the training passes: dst[r] = scale[perm[r]] * src[perm[r] / k]
 * for r < R (scale NULL: 1; perm[r] < 0: a zero row).  src device FP32 [*][d],
 * dst [R][d], perm device int32 [R] (e.g. perm_c of mm_drop_pad), scale
 * device FP32 per assignment t*k+j (e.g. the gate weights, to form the
 * expert output gradient w_tj dy_t).  d a multiple of 4.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE.
 */
mm_status mm_gather_rows(int64_t R, int64_t d, int32_t k, const int32_t* perm, const float* scale,
                         const float* src, float* dst, void* stream);

/*
 * QAT forward of the routed experts over expert-ordered rows (section
 * "Pre-training": the experts batched into grouped matrix products; eq. (6)
 * fake quantisation).  Expert e owns rows [offsets[e], offsets[e+1]) (device
 * int32 [E+1], offsets[E] = R) of xs (device FP32 [R][d], the fake-quantised
 * input rows); w_gu FP32 [E][2h][d] (gate rows first) and w_d FP32 [E][d][h]
 * are the fake-quantised weights.  Per row:
 *   gu = w_gu_e xs_r                 -> gu    [R][2h]  (FP32 matrix cores)
 *   a_bar = fake quant (b = 8, per row) of silu(g) * u  -> a_bar [R][h]
 *   f = w_d_e a_bar_r                -> f     [R][d]
 * gu and a_bar are what mm_expert_backward_f32 takes.  d, h multiples of 16.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE.
 */
mm_status mm_expert_train_forward_f32(int32_t E, int32_t d, int32_t h, int64_t R,
                                      const int32_t* offsets, const float* xs, const float* w_gu,
                                      const float* w_d, float* gu, float* a_bar, float* f,
                                      void* stream);

/* Workspace of mm_expert_backward_f32: 12 * R * h bytes (0 for invalid sizes). */
size_t mm_expert_backward_workspace_bytes(int64_t R, int32_t h);

/*
 * Backward of mm_expert_train_forward_f32 given the gradient df of the
 * expert output rows (device FP32 [R][d]) and the forward's gu and a_bar:
 *   da = (w_d_e^T df_r) * pass   (straight-through rounding; the clamp of the
 *        INT8 activation quantiser differentiated at the rounded quotient)
 *   dg = da u silu'(g), du = da silu(g)
 *   dxs   [R][d]      = w_gu_e^T [dg, du]
 *   dw_d  [E][d][h]   = sum over the expert's rows of df_r a_bar_r^T
 *   dw_gu [E][2h][d]  = sum over the expert's rows of [dg, du]_r xs_r^T
 * (experts without rows get zero weight gradients).  The gradients are with
 * respect to the fake-quantised operands; mm_fake_quant's backward carries
 * them to the latent weights and inputs.  FP32 matrix cores, FP32 sums:
 * tolerance-checked against the oracle's double evaluation.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE, MM_ERR_WORKSPACE.
 */
mm_status mm_expert_backward_f32(int32_t E, int32_t d, int32_t h, int64_t R, const int32_t* offsets,
                                 const float* xs, const float* w_gu, const float* w_d,
                                 const float* gu, const float* a_bar, const float* df, float* dxs,
                                 float* dw_gu, float* dw_d, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * Router backward of the training step (section "Pre-training", stability
 * list: FP32 router, router z-loss, softmax or sigmoid-renormalised gate by
 * desc->gating).  Inputs: x FP32 [T][d] (the router input), w_router FP32
 * [E][d], bias [E] (may be NULL), topk_idx int32 [T][k], f FP32 [*][d] the
 * expert output rows of the kept routing with inv int32 [T*k] (row, or -1
 * when dropped), dy FP32 [T][d] the gradient of the layer output.
 *   g_j = dy_t . f_inv(t,j);  z = x_t Wr^T (+ bias unless selection-only)
 *   softmax gate: dz = p * (G - <p, G>), sigmoid gate: dz_idx(j) =
 *   sig'(z)/S (g_j - sum_i w_i g_i); both plus (2 lambda_z / T) lse(z) p
 * Outputs: dz FP32 [T][E], dw_router FP32 [E][d], and dx FP32 [T][d] += dz Wr
 * (accumulated: pass the experts' token gradient, or zeros).  The bias gets
 * no gradient.  E <= 64 and a multiple of 4, d a multiple of 16.  FP32
 * arithmetic, tolerance-checked against the oracle's double evaluation.
 * Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE.
 */
mm_status mm_router_backward_f32(const mm_layer_desc* desc, int64_t T, const float* x,
                                 const float* w_router, const float* bias, const int32_t* topk_idx,
                                 const float* f, const int32_t* inv, const float* dy,
                                 float lambda_z, float* dz, float* dw_router, float* dx,
                                 void* stream);

/* Row RMSNorm with unit gain used between stacked layers of the decode
 * workload (not part of eq. (*)): y = x / sqrt(mean(x^2) + eps), FP32. */
mm_status mm_rmsnorm_f32(int64_t rows, int64_t cols, float eps, const float* x, float* y,
                         void* stream);

/*
 * The join of a decoder block's sub-layers (section "MoE preliminaries and
 * three design factors": each layer is attention plus the FFN on the
 * residual stream): sum = x + r (FP32, elementwise) and, when norm is not
 * NULL, norm = RMSNorm(sum) with eps (> 0) and unit gain, the next
 * sub-layer's input.  All device FP32 [rows][cols]; outputs must not alias
 * inputs.  Errors: MM_ERR_NULL / MM_ERR_ALIGN, MM_ERR_SHAPE.
 */
mm_status mm_add_rmsnorm_f32(int64_t rows, int64_t cols, float eps, const float* x, const float* r,
                             float* sum, float* norm, void* stream);

/*
 * Test-only twins of the INT4 gate/up and down calls that also write the
 * exact int32 group sums of the same kernels:
 *   gate/up: isum [T*k][2h][d/32] (sorted order), down: isum [T*k][d][h/32].
 */
mm_status mm_expert_gateup_swiglu_dbg(const mm_layer_desc* desc, int64_t T, const void* act,
                                      const float* act_scale, const int32_t* perm,
                                      const int32_t* expert_offsets, mm_weight w_gateup,
                                      void* h, float* h_scale, void* ws, size_t ws_bytes,
                                      int32_t* isum, void* stream);
mm_status mm_expert_down_dbg(const mm_layer_desc* desc, int64_t T, const void* h,
                             const float* h_scale, const int32_t* expert_offsets,
                             mm_weight w_down, float* f, void* ws, size_t ws_bytes,
                             int32_t* isum, void* stream);
/* ... and of the merged products: isum_r [T*k][2h][d/32] and isum_s
 * [T][2h_s][d/32] (gate/up), isum_r [T*k][d][h/32] and isum_s [T][d][h_s/32]
 * (down), each the exact group sum of one (row, weight row, group). */
mm_status mm_expert_gateup_pair_f32_dbg(const mm_layer_desc* desc, int64_t T, const void* xq,
                                        const float* sx, const int32_t* perm,
                                        const int32_t* expert_offsets, mm_weight w_gateup,
                                        mm_weight ws_gateup, float* h_r, float* h_s,
                                        int32_t* isum_r, int32_t* isum_s, void* stream);
mm_status mm_expert_down_pair_f32_dbg(const mm_layer_desc* desc, int64_t T, const void* hq_r,
                                      const float* hs_r, const void* hq_s, const float* hs_s,
                                      const int32_t* expert_offsets, mm_weight w_down,
                                      mm_weight ws_down, float* f, float* ys, int32_t* isum_r,
                                      int32_t* isum_s, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOBMOE_H */
