// Router helpers shared by the router kernels and the fused decode layer:
// the top-k selection with its gate weights, the bias handling, and the
// per-token INT8 quantisation of a row held in registers.  (MobileMoE close
// reading, section "Pre-training": FP32 router, softmax or sigmoid gate,
// load-balancing bias; section "Quantisation-aware training": INT8
// activations.)  Every function is called by a whole wave.
#pragma once

#include "common.h"

namespace mm {

// Top-k and gate weights of one token; lane e holds the logit of expert e
// (-inf for e >= E).  k rounds of a wave arg-max under the total order (value
// descending, index ascending): the round's maximum, then the lowest lane
// holding it; lane j keeps the winner of round j.  Writes idx[0..k) and
// w[0..k).  Called by a whole wave.
// gl: the logit the gate weight is computed from (mine itself, or with the
// selection-only bias the logit without that bias).  kGating & 1: sigmoid
// rule; the softmax subtracts the maximum of gl over the experts.
template <int kGating>
__device__ __forceinline__ void select_topk_lanes(float mine, float gl, int lane, int E, int k,
                                                  int& my_sel, float& wv) {
  const bool valid = lane < E;
  bool avail = valid;
  my_sel = 0;
  for (int j = 0; j < k; ++j) {
    const float mx = max64(avail ? mine : -INFINITY);
    const uint64_t hits = __ballot(avail && mine == mx);
    const int win = __ffsll((unsigned long long)hits) - 1;
    if (lane == j) my_sel = win;
    if (lane == win) avail = false;
  }
  if ((kGating & 1) == 0) {
    // softmax over all E logits, not renormalised over the k selected
    const float m = max64(valid ? gl : -INFINITY);
    const float z = valid ? exp_fp32(gl - m) : 0.0f;
    const float S = tree_sum64(z);
    wv = __shfl(z, my_sel) / S;
  } else {
    // sigmoid of each selected logit, normalised over the k selected
    const float sg = valid ? 1.0f / (1.0f + exp_fp32(-gl)) : 0.0f;
    const float mysg = __shfl(sg, my_sel);
    const float S = tree_sum64(lane < k ? mysg : 0.0f);
    wv = mysg / S;
  }
}

// Lane e's ranking value and gate logit from the stored logit without the
// bias (row[e], e < E): the ranking value is logit + bias[e] (-inf for e >=
// E); the gate logit is the same value, or with the selection-only bias
// (kGating & 2, the load-balancing bias of the "Pre-training" section) the
// logit without the bias.
template <int kGating>
__device__ __forceinline__ void biased_value(float raw, const float* __restrict__ bias, int lane,
                                             int E, float& mine, float& gl) {
  const float b = raw + (bias && lane < E ? bias[lane] : 0.0f);
  mine = lane < E ? b : -INFINITY;
  gl = (kGating & 2) ? raw : b;
}

template <int kGating>
__device__ __forceinline__ void biased_logit(const float* row, const float* __restrict__ bias,
                                             int lane, int E, float& mine, float& gl) {
  biased_value<kGating>(lane < E ? row[lane] : 0.0f, bias, lane, E, mine, gl);
}

// Per-token INT8 quantisation of the x row a wave holds in registers (lane l
// holds columns l, l + 64, ...): the same rule as the row quantiser,
// s = (2 * max|x|) / 255, q = clamp(rint(x / s)), s = 0 gives q = 0.
// gm_rows: the layout as in store_code (common.h).
template <int kNX>
__device__ __forceinline__ void quant_row_regs(const float (&xv)[kNX], int lane, int64_t t,
                                               int d, int8_t* __restrict__ xq,
                                               float* __restrict__ sx, int64_t gm_rows) {
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kNX; ++c) amax = fmaxf(amax, fabsf(xv[c]));
  amax = max64(amax);
  const float s = (2.0f * amax) / 255.0f, y = quant_recip(s);
  if (lane == 0) sx[t] = s;
#pragma unroll
  for (int c = 0; c < kNX; ++c)
    store_code(xq, t, lane + kWave * c, d, gm_rows, s != 0.0f ? quant_i8(xv[c], s, y) : 0);
}

}  // namespace mm
