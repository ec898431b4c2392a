// FP32 router: logits, top-k selection and gate weights.
//
// The router stays in FP32 (MobileMoE close reading, section "Pre-training",
// MoE stability list); eq. (*) weights each selected expert's output by
// router_i(x).  The logit of (token t, expert e) is computed in one fixed
// order so that the selection is reproducible bit for bit:
//   lane l of a wave accumulates x[t][j] * w[e][j] for j = l, l+64, ... with
//   fused multiply-adds, then the 64 partials are added as a balanced binary
//   tree over lane indices (pairs at distance 1, 2, 4, ..., 32), then bias[e]
//   is added.  Experts are ranked by (logit descending, index ascending).
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

constexpr int kMaxX = 32;   // d <= 2048 keeps the token rows in registers
constexpr int kTok = 4;     // tokens per workgroup (one per wave for the top-k)

// Workgroup = 4 waves and 4 tokens.  Phase 1: wave w computes the logits of
// experts w, w+4, w+8, ... for all 4 tokens (the expert's weight row is loaded
// once per wave and reused for the 4 tokens) into LDS.  Phase 2: wave w takes
// token w, lane e holding the logit of expert e, and does the top-k and the
// gate weights.
template <int kGating>
__global__ __launch_bounds__(256) void k_router(int64_t T, int d, int E, int k,
                                                const float* __restrict__ x,
                                                const float* __restrict__ wr,
                                                const float* __restrict__ bias,
                                                int32_t* __restrict__ idx,
                                                float* __restrict__ w) {
  __shared__ float s_logit[kTok][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int nt = (int)min((int64_t)kTok, T - t0);
  const int nx = d / kWave;

  if (nx <= kMaxX) {
    float xv[kTok][kMaxX];
#pragma unroll
    for (int q = 0; q < kTok; ++q)
#pragma unroll
      for (int i = 0; i < kMaxX; ++i)
        if (i < nx) xv[q][i] = q < nt ? x[(t0 + q) * d + lane + kWave * i] : 0.0f;
    for (int e = wave; e < E; e += 4) {
      const float* we = wr + (int64_t)e * d;
      float wv[kMaxX];
#pragma unroll
      for (int i = 0; i < kMaxX; ++i)
        if (i < nx) wv[i] = we[lane + kWave * i];
      const float b = bias ? bias[e] : 0.0f;
#pragma unroll
      for (int q = 0; q < kTok; ++q) {
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < kMaxX; ++i)
          if (i < nx) p = __builtin_fmaf(xv[q][i], wv[i], p);
        p = tree_sum64(p);
        if (lane == 0) s_logit[q][e] = p + b;
      }
    }
  } else {
    for (int e = wave; e < E; e += 4) {
      const float* we = wr + (int64_t)e * d;
      const float b = bias ? bias[e] : 0.0f;
      for (int q = 0; q < kTok; ++q) {
        float p = 0.0f;
        if (q < nt)
          for (int j = lane; j < d; j += kWave) p = __builtin_fmaf(x[(t0 + q) * d + j], we[j], p);
        p = tree_sum64(p);
        if (lane == 0) s_logit[q][e] = p + b;
      }
    }
  }
  __syncthreads();
  if (wave >= nt) return;
  const int64_t t = t0 + wave;
  const float mine = lane < E ? s_logit[wave][lane] : -INFINITY;

  // Top-k: k rounds of a wave arg-max under the total order (value
  // descending, index ascending): the round's maximum, then the lowest lane
  // holding it.  Lane j keeps the winner of round j.
  const bool valid = lane < E;
  bool avail = valid;
  int my_sel = 0;
  float m = 0.0f;
  for (int j = 0; j < k; ++j) {
    const float mx = max64(avail ? mine : -INFINITY);
    const uint64_t hits = __ballot(avail && mine == mx);
    const int win = __ffsll((unsigned long long)hits) - 1;
    if (j == 0) m = mx;
    if (lane == j) my_sel = win;
    if (lane == win) avail = false;
  }

  float wv;
  if (kGating == 0) {
    // softmax over all E logits, not renormalised over the k selected
    const float z = valid ? exp_fp32(mine - m) : 0.0f;
    const float S = tree_sum64(z);
    wv = __shfl(z, my_sel) / S;
  } else {
    // sigmoid of each selected logit, normalised over the k selected
    const float sg = valid ? 1.0f / (1.0f + exp_fp32(-mine)) : 0.0f;
    const float mysg = __shfl(sg, my_sel);
    const float S = tree_sum64(lane < k ? mysg : 0.0f);
    wv = mysg / S;
  }
  if (lane < k) {
    idx[t * k + lane] = my_sel;
    w[t * k + lane] = wv;
  }
}

}  // namespace

hipError_t launch_router(int64_t T, int d, int E, int k, int gating, const float* x,
                         const float* wr, const float* bias, int32_t* idx, float* w,
                         hipStream_t st) {
  const unsigned blocks = (unsigned)((T + kTok - 1) / kTok);
  if (gating == 0)
    hipLaunchKernelGGL(k_router<0>, dim3(blocks), dim3(256), 0, st, T, d, E, k, x, wr, bias, idx, w);
  else
    hipLaunchKernelGGL(k_router<1>, dim3(blocks), dim3(256), 0, st, T, d, E, k, x, wr, bias, idx, w);
  return hipGetLastError();
}

}  // namespace mm
