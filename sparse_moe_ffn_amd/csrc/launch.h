// Host-side launchers of the libmobmoe kernels.  Each returns the result of
// hipGetLastError() after queueing its kernels on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace mm {

// Layouts of the INT8 activation codes a quantiser writes (common.h):
// row-major int8, group-major int8, or f16 paired (2 bytes per code, the
// operand form of the f16 matrix-core products).
enum ActLayout : int { kActRowMajor = 0, kActGroupMajor = 1, kActF16Paired = 2 };
// gm_rows argument of the device code for a matrix of `rows` rows.
inline int64_t act_gm_rows(int layout, int64_t rows) {
  return layout == kActGroupMajor ? rows : layout == kActF16Paired ? kF16Paired : 0;
}

// Quantisation, packing, conversions (k_quant.hip)
hipError_t launch_quantize_int4g32(int64_t rows, int64_t cols, const float* w, uint8_t* q,
                                   float* s, hipStream_t st);
hipError_t launch_prepack_int4g32(int64_t n_mat, int64_t rows, int64_t cols, const uint8_t* qc,
                                  const float* sc, uint8_t* qo, float* so, hipStream_t st);
// layout: ActLayout of the codes (group-major and f16 paired: cols % 128 == 0
// only); q holds rows * cols bytes, twice that for f16 paired.
hipError_t launch_act_quant_i8(int64_t rows, int64_t cols, const float* x, int8_t* q, float* s,
                               hipStream_t st, int layout = kActRowMajor);
// Two row sets (e.g. the routed and the shared hidden rows) in one launch.
hipError_t launch_act_quant_i8_pair(int64_t rows0, int64_t cols0, const float* x0, int8_t* q0,
                                    float* s0, int64_t rows1, int64_t cols1, const float* x1,
                                    int8_t* q1, float* s1, hipStream_t st, int layout = kActRowMajor);
hipError_t launch_convert_bf16(int64_t n, const float* x, uint16_t* y, hipStream_t st);
hipError_t launch_rmsnorm(int64_t rows, int64_t cols, float eps, const float* x, float* y,
                          hipStream_t st);
// sum = x + r; norm (may be null) = RMSNorm(sum) with eps, unit gain.
hipError_t launch_add_rmsnorm(int64_t rows, int64_t cols, float eps, const float* x,
                              const float* r, float* sum, float* norm, hipStream_t st);

// Router (k_router.hip)
// xq / sx non-null: also the per-token INT8 quantisation of x (in the same
// pass where the width has a register form, else a second kernel).
hipError_t launch_router(int64_t T, int d, int E, int k, int gating, const float* x,
                         const float* wr, const float* bias, int32_t* idx, float* w,
                         int8_t* xq, float* sx, hipStream_t st, int xq_layout = kActRowMajor,
                         uint8_t* hist = nullptr, int64_t hist_stride = 0);
// hist (T > 64 only): each 4-token router workgroup's count of every expert,
// byte hist[e * hist_stride + b], b < ceil(T / 4); input of launch_route_hist.

// Router + top-k + INT8 of x + the count sort in one workgroup, for
// 1 <= T <= 2 tokens (beyond that the per-token router workgroups win) and
// the widths with a register form up to d = 1280
// (k_router.hip).  Returns false (nothing launched) otherwise.  Outputs as
// launch_router (with xq / sx) followed by launch_route.
bool launch_front_small(int64_t T, int d, int E, int k, int gating, const float* x,
                        const float* wr, const float* bias, int32_t* idx, float* w, int8_t* xq,
                        float* sx, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                        hipStream_t st);

// Route / permute (k_route.hip).  ws holds ceil(T*k/256) * E int32 counts.
int64_t route_blocks(int64_t Tk);
// Count sort from the router's per-workgroup expert counts (launch_router
// with hist): one kernel instead of two.  hist holds E rows of
// route_hist_stride(T) bytes.
int64_t route_hist_stride(int64_t T);
bool route_hist_applies(int64_t T, int k);
hipError_t launch_route_hist(int64_t T, int k, int E, const int32_t* idx, const uint8_t* hist,
                             int32_t* offsets, int32_t* perm, int32_t* inv_perm, hipStream_t st);
hipError_t launch_route(int64_t Tk, int E, const int32_t* idx, int32_t* offsets, int32_t* perm,
                        int32_t* inv_perm, int32_t* ws, hipStream_t st);

// Expert products (k_expert.hip).  `perm`/`offsets` are null for the dense
// (shared-expert) form, where the rows are the T tokens in order.
struct ExpertArgs {
  int64_t rows;        // routed: T*k sorted positions; dense: T
  int64_t T;           // tokens
  int d, h, E, k;      // h = hidden of this expert kind
  const int32_t* perm;
  const int32_t* offsets;
};
// Grid size in tiles of bm rows: dense ceil(rows / bm); routed (tiles per
// expert from the offsets, known only on the device) the bound ceil(rows /
// bm) + min(E, rows): every expert that owns rows adds at most one partial
// tile, and at most min(E, rows) experts own rows.
inline int64_t tile_bound(const ExpertArgs& a, int64_t bm) {
  const int64_t full = (a.rows + bm - 1) / bm;
  return a.offsets ? full + (a.rows < a.E ? a.rows : (int64_t)a.E) : full;
}
// INT4 gate/up + SwiGLU + per-row INT8 re-quantisation: hq [rows][h], hs [rows].
// a_buf [rows][h] FP32 is staging space for the unquantised hidden rows.
hipError_t launch_gateup_i4(const ExpertArgs& a, const int8_t* xq, const float* sx,
                            const uint8_t* wq, const float* ws, float* a_buf, int8_t* hq,
                            float* hs, int32_t* isum, hipStream_t st);
// INT4 down: f [rows][d] = s_h * sum_g s_w * isum_g
hipError_t launch_down_i4(const ExpertArgs& a, const int8_t* hq, const float* hs,
                          const uint8_t* wq, const float* ws, float* f, int32_t* isum,
                          hipStream_t st);
// Matrix-core forms (k_mfma.hip) for larger row counts.  Gate/up writes the
// FP32 hidden rows a = SiLU(g) * u to a_buf [rows][h]; re-quantise them with
// launch_act_quant_i8.  Down writes f [rows][d].
hipError_t launch_gateup_i4_mfma(const ExpertArgs& a, const int8_t* xq, const float* sx,
                                 const uint8_t* wq, const float* ws, float* a_buf, int32_t* isum,
                                 hipStream_t st);
hipError_t launch_down_i4_mfma(const ExpertArgs& a, const int8_t* hq, const float* hs,
                               const uint8_t* wq, const float* ws, float* f, int32_t* isum,
                               hipStream_t st);
// Weight-streaming forms (k_gemv.hip) for a few rows per expert: same
// outputs as the matrix-core forms (gate/up: FP32 hidden rows to a_buf).  gemv_i4_fits(K, gateup) tells whether a
// reduction length is supported (K % 64 == 0, K <= 2560, LDS within 64 KB).
bool gemv_i4_fits(int K, bool gateup);
hipError_t launch_gateup_i4_gemv(const ExpertArgs& a, const int8_t* xq, const float* sx,
                                 const uint8_t* wq, const float* ws, float* a_buf, int32_t* isum,
                                 hipStream_t st);
hipError_t launch_down_i4_gemv(const ExpertArgs& a, const int8_t* hq, const float* hs,
                               const uint8_t* wq, const float* ws, float* f, int32_t* isum,
                               hipStream_t st);
// Weight-streaming forms are used up to this many rows (routed: all experts
// together; dense: the tokens): decode batches up to 8 tokens of top-4.
// Beyond that the one-wave matrix-core tiles are faster even with most of
// their 32 rows padding (S decode stack: B = 16 -11 %, 32 -21 %, 64 -35 %;
// L layer at B = 64 -60 %): the weight-streaming kernels' dot products grow
// with the rows of a tile, and an expert with more than four rows has its
// weights read once per four.
constexpr int64_t kGemvMaxRowsRouted = 32;
constexpr int64_t kGemvMaxRowsDense = 8;
// The matrix-core forms are used from this many rows on, when the reduction
// dimension is a multiple of 128.
constexpr int64_t kMfmaMinRows = kGemvMaxRowsRouted + 1;
// Routed and shared products of one kind in a single launch: matrix-core
// and weight-streaming forms.  The matrix-core pair reads its INT8
// activations (x_q [T][d] for gate/up; the hidden rows [Tk][h], [T][hs] for
// down) in the group-major layout; the weight-streaming pair reads them
// row-major.
hipError_t launch_gateup_i4_mfma_pair(const ExpertArgs& ar, const ExpertArgs& as,
                                      const int8_t* xq, const float* sx, const uint8_t* wq_r,
                                      const float* ws_r, const uint8_t* wq_s, const float* ws_s,
                                      float* abuf_r, float* abuf_s, hipStream_t st);
hipError_t launch_down_i4_mfma_pair(const ExpertArgs& ar, const ExpertArgs& as,
                                    const int8_t* hq_r, const float* hs_r, const int8_t* hq_s,
                                    const float* hs_s, const uint8_t* wq_r, const float* ws_r,
                                    const uint8_t* wq_s, const float* ws_s, float* f, float* ys,
                                    hipStream_t st);
// The same two products with the weighted combine in the shared down's
// epilogue (y [T][d] written, no ys): the routed down first, then the shared
// down, whose tiles gather each token's routed outputs through inv_perm and
// add them, weighted by topk_w, in the combine's order.  down_cmb_fits: k <= 8,
// d % 64 == 0, one shared row per token, and enough tokens (4096) that this
// form is the faster one.
bool down_cmb_fits(const ExpertArgs& ar, const ExpertArgs& as);
hipError_t launch_down_i4_mfma_cmb(const ExpertArgs& ar, const ExpertArgs& as, const int8_t* hq_r,
                                   const float* hs_r, const int8_t* hq_s, const float* hs_s,
                                   const uint8_t* wq_r, const float* ws_r, const uint8_t* wq_s,
                                   const float* ws_s, float* f, const int32_t* inv_perm,
                                   const float* topk_w, float* y, hipStream_t st);
hipError_t launch_gateup_i4_gemv_pair(const ExpertArgs& ar, const ExpertArgs& as,
                                      const int8_t* xq, const float* sx, const uint8_t* wq_r,
                                      const float* ws_r, const uint8_t* wq_s, const float* ws_s,
                                      float* abuf_r, float* abuf_s, hipStream_t st);
hipError_t launch_down_i4_gemv_pair(const ExpertArgs& ar, const ExpertArgs& as,
                                    const int8_t* hq_r, const float* hs_r, const int8_t* hq_s,
                                    const float* hs_s, const uint8_t* wq_r, const float* ws_r,
                                    const uint8_t* wq_s, const float* ws_s, float* f, float* ys,
                                    hipStream_t st);
// Same pair from the FP32 hidden rows a_r [Tk][h], a_s [T][hs]: each
// workgroup quantises its rows itself (codes and scales bit-identical to
// launch_act_quant_i8_pair), so no quantiser launch is needed.  Only when
// gemv_i4_qin_fits(h) and gemv_i4_qin_fits(hs).
bool gemv_i4_qin_fits(int K);
hipError_t launch_down_i4_gemv_pair_f32in(const ExpertArgs& ar, const ExpertArgs& as,
                                          const float* a_r, const float* a_s, const uint8_t* wq_r,
                                          const float* ws_r, const uint8_t* wq_s,
                                          const float* ws_s, float* f, float* ys, hipStream_t st);
constexpr int kMfmaK = 128;
// The same pairs on the f16 matrix cores with exact group sums (k_w4f16.hip):
// activations as f16 paired codes (x16 [T][d]; the hidden rows h16_r [Tk][h],
// h16_s [T][hs]); bit-identical outputs.  isum_r / isum_s non-null (tests):
// also the exact group sums [rows][wrows][K / 32].  f16_products_fit: widths
// they take (K % 64 == 0, h and hs % 64 == 0, d % 128 == 0).
bool f16_products_fit(int d, int h, int hs);
hipError_t launch_gateup_f16_pair(const ExpertArgs& ar, const ExpertArgs& as, const uint16_t* x16,
                                  const float* sx, const uint8_t* wq_r, const float* ws_r,
                                  const uint8_t* wq_s, const float* ws_s, float* abuf_r,
                                  float* abuf_s, int32_t* isum_r, int32_t* isum_s,
                                  hipStream_t st);
hipError_t launch_down_f16_pair(const ExpertArgs& ar, const ExpertArgs& as, const uint16_t* h16_r,
                                const float* hs_r, const uint16_t* h16_s, const float* hs_s,
                                const uint8_t* wq_r, const float* ws_r, const uint8_t* wq_s,
                                const float* ws_s, float* f, float* ys, int32_t* isum_r,
                                int32_t* isum_s, hipStream_t st);
// BF16 weights on the bf16 matrix cores (k_bf16.hip): gate/up takes the
// token rows already rounded to BF16 (xb [T][d]) and writes BF16 hidden rows
// [rows][h]; down writes f [rows][d] FP32.
hipError_t launch_gateup_bf16_mfma(const ExpertArgs& a, const uint16_t* xb, const uint16_t* w,
                                   uint16_t* h_out, hipStream_t st);
hipError_t launch_down_bf16_mfma(const ExpertArgs& a, const uint16_t* hb, const uint16_t* w,
                                 float* f, hipStream_t st);
// Floating-point row-tile forms: bf16 = false uses FP32 operands, true uses BF16.
hipError_t launch_gateup_fp(const ExpertArgs& a, bool bf16, const void* x, const void* w,
                            void* h_out, hipStream_t st);
hipError_t launch_down_fp(const ExpertArgs& a, bool bf16, const void* hrow, const void* w,
                          float* f, hipStream_t st);

// Combine (k_combine.hip)
// y_norm non-null (FP32 y only): also RMSNorm(y) with eps, unit gain.
hipError_t launch_combine(int64_t T, int d, int k, const float* f, const int32_t* inv_perm,
                          const float* w, const float* ys, void* y, bool bf16_out,
                          hipStream_t st, float* y_norm = nullptr, float eps = 0.0f);

// The whole layer for 1..4 tokens in one launch (k_decode.hip), INT4
// weights; the same outputs as the separate launches.  state: a block of
// decode_fused_state_bytes() (call count, exit counter, logit table), and
// a_r / a_s / f / ys, zeroed before first use; each call leaves them ready
// for the next (word 4 of the state counts waits that gave up).  grid_out: the
// launched workgroup count.  hipErrorInvalidConfiguration if the grid cannot
// be resident at once.
struct DecodeFusedArgs {
  int64_t T;
  int d, E, k, h, hs, gating;
  const float* x;
  const float* wr;
  const float* bias;
  const uint8_t* gq;
  const float* gs;
  const uint8_t* dq;
  const float* ds;
  const uint8_t* sgq;
  const float* sgs;
  const uint8_t* sdq;
  const float* sds;
  int32_t* topk_idx;
  float* topk_w;
  void* y;
  float* y_norm;
  float eps;
  bool out_bf16;
  void* state;
  void* a_r;  // flag-in-word buffers: 8 bytes per value
  void* a_s;
  void* f;
  void* ys;
  uint32_t spin_limit;
};
bool decode_fused_fits(int64_t T, int d, int E, int k, int h, int hs);
size_t decode_fused_state_bytes();
hipError_t launch_decode_fused(const DecodeFusedArgs& a, hipStream_t st, int* grid_out = nullptr);
// The no-allocation form's device scratch (k_decode.hip): its size, and its
// address on the current device (looked up, and its state block cleared on
// stream st, at the first call per device).
size_t decode_scratch_capacity();
hipError_t decode_scratch(void** out, hipStream_t st);

// Decode attention over an INT8 KV cache (k_attn.hip).  Head width 64, up
// to 8 query heads per key/value head.
size_t attn_partial_bytes(int64_t B, int nkv, int64_t max_len);
hipError_t launch_kv_append(int64_t B, int nkv, int64_t maxT, const int32_t* pos,
                            const float* k_new, const float* v_new, int8_t* kc, int8_t* vc,
                            float* ks, float* vs, hipStream_t st);
hipError_t launch_attn_decode(int64_t B, int nh, int nkv, int64_t maxT, int64_t max_len,
                              const int32_t* lens, const float* q, const int8_t* kc,
                              const int8_t* vc, const float* ks, const float* vs, float* part,
                              float* out, hipStream_t st);

}  // namespace mm
