// FP32 router: logits, top-k selection and gate weights.
//
// The router stays in FP32 (MobileMoE close reading, section "Pre-training",
// MoE stability list); eq. (*) weights each selected expert's output by
// router_i(x).  The logit of (token t, expert e) is computed in one fixed
// order so that the selection is reproducible bit for bit:
//   lane l of a wave accumulates x[t][j] * w[e][j] for j = l, l+64, ... with
//   fused multiply-adds, then the 64 partials are added as a balanced binary
//   tree (xor-butterfly with distances 1, 2, 4, 8, 16, 32; every lane ends with
//   the same value because IEEE addition is commutative), then bias[e] is
//   added.  Experts are ranked by (logit descending, index ascending).
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

constexpr int kMaxXRegs = 32;  // d <= 2048 keeps the token row in registers

// One wave per token, lanes 0..E-1 end up owning the logits of experts 0..E-1.
template <int kGating>
__global__ __launch_bounds__(256) void k_router(int64_t T, int d, int E, int k,
                                                const float* __restrict__ x,
                                                const float* __restrict__ wr,
                                                const float* __restrict__ bias,
                                                int32_t* __restrict__ idx,
                                                float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* xr = x + t * d;
  const int nx = d / kWave;

  float xv[kMaxXRegs];
  if (nx <= kMaxXRegs) {
#pragma unroll
    for (int i = 0; i < kMaxXRegs; ++i)
      if (i < nx) xv[i] = xr[lane + kWave * i];
  }

  float mine = -INFINITY;
  for (int e = 0; e < E; ++e) {
    const float* we = wr + (int64_t)e * d;
    float p = 0.0f;
    if (nx <= kMaxXRegs) {
#pragma unroll
      for (int i = 0; i < kMaxXRegs; ++i)
        if (i < nx) p = __builtin_fmaf(xv[i], we[lane + kWave * i], p);
    } else {
      for (int j = lane; j < d; j += kWave) p = __builtin_fmaf(xr[j], we[j], p);
    }
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) p = p + __shfl_xor(p, s);
    const float lg = p + (bias ? bias[e] : 0.0f);
    if (lane == e) mine = lg;
  }

  // Top-k: k rounds of a wave arg-max under the total order
  // (value descending, index ascending), removing each winner.  Lane j keeps
  // the winner of round j.
  const bool valid = lane < E;
  bool avail = valid;
  int my_sel = 0;
  float m = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = avail ? mine : -INFINITY;
    int bi = avail ? lane : 1 << 20;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      const float ov = __shfl_xor(bv, s);
      const int oi = __shfl_xor(bi, s);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (j == 0) m = bv;
    if (lane == j) my_sel = bi;
    if (lane == bi) avail = false;
  }

  float wv;
  if (kGating == 0) {
    // softmax over all E logits, not renormalised over the k selected
    const float z = valid ? __expf(mine - m) : 0.0f;
    const float S = wave_sum(z);
    wv = __shfl(z, my_sel) / S;
  } else {
    // sigmoid of each selected logit, normalised over the k selected
    const float sg = valid ? 1.0f / (1.0f + __expf(-mine)) : 0.0f;
    const float mysg = __shfl(sg, my_sel);
    const float S = wave_sum(lane < k ? mysg : 0.0f);
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
  const unsigned blocks = (unsigned)((T + 3) / 4);
  if (gating == 0)
    hipLaunchKernelGGL(k_router<0>, dim3(blocks), dim3(256), 0, st, T, d, E, k, x, wr, bias, idx, w);
  else
    hipLaunchKernelGGL(k_router<1>, dim3(blocks), dim3(256), 0, st, T, d, E, k, x, wr, bias, idx, w);
  return hipGetLastError();
}

}  // namespace mm
