// One token's weighted combine through the inverse permutation (MobileMoE
// close reading, section "Custom MoE kernel": the expert outputs are gathered
// back to token order, weighted by the gate), the body of the combine kernel:
//   y[t][c] = fma(w[t][k-1], f[inv[t*k+k-1]][c], ... fma(w[t][0], f[inv[t*k]][c], 0))
//             + ys[t][c]
// and with kNorm also RMSNorm(y) = y / sqrt(mean(y^2) + eps) (FP32 y only;
// the input of the next layer of a decoder stack) into y_norm and/or the
// workgroup-memory row norm_lds (either may be NULL).  One wave: lane l handles the float4 columns
// l, l + 64, ... (kC4 of them); the gathers of up to four expert rows and the
// shared row are issued before the first sum.  y may be NULL (FP32 output
// not wanted).
#pragma once

#include "common.h"

namespace mm {

template <int kC4, bool kBF16Out, bool kNorm>
__device__ __forceinline__ void combine_token(int64_t t, int64_t T, int d, int k,
                                              const float* __restrict__ f,
                                              const int32_t* __restrict__ inv,
                                              const float* __restrict__ w,
                                              const float* __restrict__ ys,
                                              void* __restrict__ y, float* __restrict__ y_norm,
                                              float eps, float* __restrict__ norm_lds) {
  const int lane = threadIdx.x & 63;
  const int q = d / 4;
  const int64_t Tk = T * k;
  int my_p = -1;
  float my_w = 0.0f;
  if (lane < k) {
    const int64_t p = inv[t * k + lane];
    if (p >= 0 && p < Tk) my_p = (int)p;  // a corrupt inverse permutation reads nothing
    my_w = w[t * k + lane];
  }
  float4 sv[kC4];
  if (ys) {
#pragma unroll
    for (int i = 0; i < kC4; ++i)
      if (lane + 64 * i < q) sv[i] = reinterpret_cast<const float4*>(ys + t * d)[lane + 64 * i];
  }
  float4 acc[kC4];
#pragma unroll
  for (int i = 0; i < kC4; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (Tk <= 4) {
    // every row of f fits the four row buffers (one token): read them all
    // before the positions arrive, then take row inv[t*k+j] for j ascending
    // (rows past the last are read as row 0: valid, never taken)
    float4 v0[kC4], v1[kC4], v2[kC4], v3[kC4];
    const float4* f4 = reinterpret_cast<const float4*>(f);
    const int q1 = Tk > 1 ? q : 0, q2 = Tk > 2 ? 2 * q : 0, q3 = Tk > 3 ? 3 * q : 0;
#pragma unroll
    for (int i = 0; i < kC4; ++i) {
      const int c = min(lane + 64 * i, q - 1);
      v0[i] = f4[c];
      v1[i] = f4[q1 + c];
      v2[i] = f4[q2 + c];
      v3[i] = f4[q3 + c];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = j < k ? __shfl(my_p, j) : -1;
      const float wj = __shfl(my_w, j & 63);
      if (p < 0) continue;
      // p is the same on every lane: a branch, not a select per element
      auto fma_row = [&](const float4 (&u)[kC4]) {
#pragma unroll
        for (int i = 0; i < kC4; ++i) {
          acc[i].x = fmaf(wj, u[i].x, acc[i].x);
          acc[i].y = fmaf(wj, u[i].y, acc[i].y);
          acc[i].z = fmaf(wj, u[i].z, acc[i].z);
          acc[i].w = fmaf(wj, u[i].w, acc[i].w);
        }
      };
      if (p == 0) fma_row(v0);
      else if (p == 1) fma_row(v1);
      else if (p == 2) fma_row(v2);
      else fma_row(v3);
    }
  } else
  for (int j0 = 0; j0 < k; j0 += 4) {
    int pj[4];
    float wj[4];
    float4 v[4][kC4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      pj[jj] = j0 + jj < k ? __shfl(my_p, j0 + jj) : -1;
      wj[jj] = __shfl(my_w, j0 + jj);
      if (pj[jj] < 0) continue;
      const float4* fr = reinterpret_cast<const float4*>(f + (int64_t)pj[jj] * d);
#pragma unroll
      for (int i = 0; i < kC4; ++i)
        if (lane + 64 * i < q) v[jj][i] = fr[lane + 64 * i];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (pj[jj] < 0) continue;
#pragma unroll
      for (int i = 0; i < kC4; ++i)
        if (lane + 64 * i < q) {
          acc[i].x = fmaf(wj[jj], v[jj][i].x, acc[i].x);
          acc[i].y = fmaf(wj[jj], v[jj][i].y, acc[i].y);
          acc[i].z = fmaf(wj[jj], v[jj][i].z, acc[i].z);
          acc[i].w = fmaf(wj[jj], v[jj][i].w, acc[i].w);
        }
    }
  }
#pragma unroll
  for (int i = 0; i < kC4; ++i) {
    const int c4 = lane + 64 * i;
    if (c4 >= q) continue;
    float4 a = acc[i];
    if (ys) {
      a.x += sv[i].x;
      a.y += sv[i].y;
      a.z += sv[i].z;
      a.w += sv[i].w;
    }
    acc[i] = a;
    if (kBF16Out) {
      ushort4 o;
      o.x = f32_to_bf16(a.x);
      o.y = f32_to_bf16(a.y);
      o.z = f32_to_bf16(a.z);
      o.w = f32_to_bf16(a.w);
      reinterpret_cast<ushort4*>(y)[t * q + c4] = o;
    } else if (y != nullptr) {
      reinterpret_cast<float4*>(y)[t * q + c4] = a;
    }
  }
  if constexpr (kNorm) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kC4; ++i)
      if (lane + 64 * i < q) {
        ss = fmaf(acc[i].x, acc[i].x, ss);
        ss = fmaf(acc[i].y, acc[i].y, ss);
        ss = fmaf(acc[i].z, acc[i].z, ss);
        ss = fmaf(acc[i].w, acc[i].w, ss);
      }
    ss = wave_sum(ss);
    const float inv_rms = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < kC4; ++i) {
      const int c4 = lane + 64 * i;
      if (c4 >= q) continue;
      const float4 a = acc[i];
      const float4 o = make_float4(a.x * inv_rms, a.y * inv_rms, a.z * inv_rms, a.w * inv_rms);
      if (y_norm != nullptr) reinterpret_cast<float4*>(y_norm)[t * q + c4] = o;
      if (norm_lds != nullptr) reinterpret_cast<float4*>(norm_lds)[c4] = o;
    }
  }
}


}  // namespace mm
