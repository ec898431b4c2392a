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

constexpr int kTok = 4;     // tokens per workgroup (one per wave for the top-k)
constexpr int kRowStride = 65;  // LDS stride of one row of 64 lane partials (padded)

// Workgroup = 4 waves and 4 tokens.  Phase 1: wave w takes experts w, w+4,
// w+8, ... (at most 16); for each one, lane l forms the 4 tokens' partial sums
// over columns j = l, l+64, ... (fused multiply-adds, ascending j) and stores
// them to LDS.  Phase 2: lane r of the wave adds the 64 partials of row r
// (one (token, expert) pair) as the balanced tree, adds the bias and writes
// the logit.  Phase 3: wave w takes token w, lane e holding the logit of
// expert e, and does the top-k and the gate weights.
// kNX = d / 64 (0: any d, row read from memory in the loop).
template <int kGating, int kNX>
__global__ __launch_bounds__(256) void k_router(int64_t T, int d, int E, int k,
                                                const float* __restrict__ x,
                                                const float* __restrict__ wr,
                                                const float* __restrict__ bias,
                                                int32_t* __restrict__ idx,
                                                float* __restrict__ w) {
  __shared__ float s_part[4][16 * kTok][kRowStride];
  __shared__ float s_logit[kTok][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int nt = (int)min((int64_t)kTok, T - t0);
  const int ne = (E - wave + 3) / 4;  // experts of this wave

  if constexpr (kNX > 0) {
    float xv[kTok][kNX];
#pragma unroll
    for (int q = 0; q < kTok; ++q)
#pragma unroll
      for (int i = 0; i < kNX; ++i) xv[q][i] = q < nt ? x[(t0 + q) * d + lane + kWave * i] : 0.0f;
    // expert rows read one ahead (two register sets in ping-pong)
    float wa[kNX], wb[kNX];
    auto load_row = [&](int i, float (&wv)[kNX]) {
      const float* we = wr + (int64_t)min(wave + 4 * i, E - 1) * d;
#pragma unroll
      for (int c = 0; c < kNX; ++c) wv[c] = we[lane + kWave * c];
    };
    auto partials = [&](int i, const float (&wv)[kNX]) {
#pragma unroll
      for (int q = 0; q < kTok; ++q) {
        float p = 0.0f;
#pragma unroll
        for (int c = 0; c < kNX; ++c) p = __builtin_fmaf(xv[q][c], wv[c], p);
        s_part[wave][i * kTok + q][lane] = p;
      }
    };
    load_row(0, wa);
    for (int i = 0; i < ne; i += 2) {
      load_row(i + 1, wb);
      partials(i, wa);
      if (i + 1 >= ne) break;
      load_row(i + 2, wa);
      partials(i + 1, wb);
    }
  } else {
    for (int i = 0; i < ne; ++i) {
      const float* we = wr + (int64_t)(wave + 4 * i) * d;
      for (int q = 0; q < kTok; ++q) {
        float p = 0.0f;
        if (q < nt)
          for (int j = lane; j < d; j += kWave) p = __builtin_fmaf(x[(t0 + q) * d + j], we[j], p);
        s_part[wave][i * kTok + q][lane] = p;
      }
    }
  }
  __syncthreads();
  // Phase 2: lane r reduces row r = (expert slot i, token q) of its wave.
  if (lane < ne * kTok) {
    const float* row = s_part[wave][lane];
    float p[64];
#pragma unroll
    for (int l = 0; l < 64; ++l) p[l] = row[l];
#pragma unroll
    for (int s2 = 1; s2 < 64; s2 <<= 1)
#pragma unroll
      for (int l = 0; l < 64; l += 2 * s2) p[l] = p[l] + p[l + s2];
    const int i = lane / kTok, q = lane % kTok;
    const int e = wave + 4 * i;
    s_logit[q][e] = p[0] + (bias ? bias[e] : 0.0f);
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
  const dim3 grid((unsigned)((T + kTok - 1) / kTok)), block(256);
#define MM_ROUTER(G, NX) hipLaunchKernelGGL((k_router<G, NX>), grid, block, 0, st, T, d, E, k, x, wr, bias, idx, w)
#define MM_ROUTER_NX(G)                 \
  switch (d / kWave) {                  \
    case 4: MM_ROUTER(G, 4); break;     \
    case 8: MM_ROUTER(G, 8); break;     \
    case 12: MM_ROUTER(G, 12); break;   \
    case 16: MM_ROUTER(G, 16); break;   \
    case 20: MM_ROUTER(G, 20); break;   \
    case 24: MM_ROUTER(G, 24); break;   \
    case 32: MM_ROUTER(G, 32); break;   \
    default: MM_ROUTER(G, 0); break;    \
  }
  if (gating == 0) {
    MM_ROUTER_NX(0)
  } else {
    MM_ROUTER_NX(1)
  }
#undef MM_ROUTER_NX
#undef MM_ROUTER
  return hipGetLastError();
}

}  // namespace mm
