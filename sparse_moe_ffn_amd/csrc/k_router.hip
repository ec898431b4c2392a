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
constexpr int64_t kSmallRouterT = 64;  // up to this many tokens: the one-token-per-workgroup form

// Top-k and gate weights of one token; lane e holds the logit of expert e
// (-inf for e >= E).  k rounds of a wave arg-max under the total order (value
// descending, index ascending): the round's maximum, then the lowest lane
// holding it; lane j keeps the winner of round j.  Writes idx[0..k) and
// w[0..k).  Called by a whole wave.
template <int kGating>
__device__ __forceinline__ void select_topk(float mine, int lane, int E, int k,
                                            int32_t* __restrict__ idx, float* __restrict__ w) {
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
    idx[lane] = my_sel;
    w[lane] = wv;
  }
}

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
    // expert rows read four ahead (a ring of four register sets); rows past
    // this wave's last expert re-read expert E-1 (valid, unused)
    float wv[4][kNX];
    auto load_row = [&](int i, float (&dst)[kNX]) {
      const float* we = wr + (int64_t)min(wave + 4 * i, E - 1) * d;
#pragma unroll
      for (int c = 0; c < kNX; ++c) dst[c] = we[lane + kWave * c];
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) load_row(i, wv[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < ne) {
#pragma unroll
        for (int q = 0; q < kTok; ++q) {
          float p = 0.0f;
#pragma unroll
          for (int c = 0; c < kNX; ++c) p = __builtin_fmaf(xv[q][c], wv[i % 4][c], p);
          s_part[wave][i * kTok + q][lane] = p;
        }
      }
      if (i + 4 < 16) load_row(i + 4, wv[i % 4]);
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
  select_topk<kGating>(mine, lane, E, k, idx + t * k, w + t * k);
}

// Few tokens (decode): one token per workgroup of 16 waves; wave w takes
// experts w, w+16, w+32, w+48 and reads all of their rows at once, so the
// router costs about one memory round trip.  Each logit is the 64-lane tree
// sum of its partials (the same order as above) plus the bias.
constexpr int kSmallWaves = 16;
constexpr int kSmallPer = 4;  // experts per wave (E <= 64)

template <int kGating, int kNX>
__global__ __launch_bounds__(64 * kSmallWaves) void k_router_small(
    int64_t T, int d, int E, int k, const float* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, int32_t* __restrict__ idx, float* __restrict__ w) {
  __shared__ float s_logit[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.x;
  float xv[kNX], wv[kSmallPer][kNX];
#pragma unroll
  for (int i = 0; i < kSmallPer; ++i) {
    const float* we = wr + (int64_t)min(wave + kSmallWaves * i, E - 1) * d;
#pragma unroll
    for (int c = 0; c < kNX; ++c) wv[i][c] = we[lane + kWave * c];
  }
#pragma unroll
  for (int c = 0; c < kNX; ++c) xv[c] = x[t * d + lane + kWave * c];
#pragma unroll
  for (int i = 0; i < kSmallPer; ++i) {
    const int e = wave + kSmallWaves * i;
    if (e >= E) break;
    float p = 0.0f;
#pragma unroll
    for (int c = 0; c < kNX; ++c) p = __builtin_fmaf(xv[c], wv[i][c], p);
    const float l = tree_sum64(p) + (bias ? bias[e] : 0.0f);
    if (lane == 0) s_logit[e] = l;
  }
  __syncthreads();
  if (wave != 0) return;
  const float mine = lane < E ? s_logit[lane] : -INFINITY;
  select_topk<kGating>(mine, lane, E, k, idx + t * k, w + t * k);
}

template <int kG, int kNX>
void launch_router_nx(bool small, int64_t T, int d, int E, int k, const float* x, const float* wr,
                      const float* bias, int32_t* idx, float* w, hipStream_t st) {
  if constexpr (kNX > 0 && kNX <= 20) {
    if (small) {
      hipLaunchKernelGGL((k_router_small<kG, kNX>), dim3((unsigned)T), dim3(64 * kSmallWaves), 0,
                         st, T, d, E, k, x, wr, bias, idx, w);
      return;
    }
  }
  hipLaunchKernelGGL((k_router<kG, kNX>), dim3((unsigned)((T + kTok - 1) / kTok)), dim3(256), 0,
                     st, T, d, E, k, x, wr, bias, idx, w);
}

template <int kG>
void launch_router_g(bool small, int64_t T, int d, int E, int k, const float* x, const float* wr,
                     const float* bias, int32_t* idx, float* w, hipStream_t st) {
  switch (d % kWave == 0 ? d / kWave : 0) {
    case 4: launch_router_nx<kG, 4>(small, T, d, E, k, x, wr, bias, idx, w, st); break;
    case 8: launch_router_nx<kG, 8>(small, T, d, E, k, x, wr, bias, idx, w, st); break;
    case 12: launch_router_nx<kG, 12>(small, T, d, E, k, x, wr, bias, idx, w, st); break;
    case 16: launch_router_nx<kG, 16>(small, T, d, E, k, x, wr, bias, idx, w, st); break;
    case 20: launch_router_nx<kG, 20>(small, T, d, E, k, x, wr, bias, idx, w, st); break;
    case 24: launch_router_nx<kG, 24>(small, T, d, E, k, x, wr, bias, idx, w, st); break;
    case 32: launch_router_nx<kG, 32>(small, T, d, E, k, x, wr, bias, idx, w, st); break;
    default: launch_router_nx<kG, 0>(small, T, d, E, k, x, wr, bias, idx, w, st); break;
  }
}

}  // namespace

hipError_t launch_router(int64_t T, int d, int E, int k, int gating, const float* x,
                         const float* wr, const float* bias, int32_t* idx, float* w,
                         hipStream_t st) {
  // few tokens: one 16-wave workgroup per token (widths with a register form up to 1280)
  const bool small = T <= kSmallRouterT;
  if (gating == 0)
    launch_router_g<0>(small, T, d, E, k, x, wr, bias, idx, w, st);
  else
    launch_router_g<1>(small, T, d, E, k, x, wr, bias, idx, w, st);
  return hipGetLastError();
}

}  // namespace mm
