// Weighted combine through the inverse permutation (MobileMoE close reading,
// section "Custom MoE kernel": expert outputs are scattered back to token
// order, weighted by the gate).  Written as a gather so that no two threads
// write the same output and no atomics are needed:
//   y[t][c] = fma(w[t][k-1], f[inv[t*k+k-1]][c], ... fma(w[t][0], f[inv[t*k]][c], 0))
//             + ys[t][c]
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

// One thread per (token, 4 consecutive columns).
template <bool kBF16Out>
__global__ __launch_bounds__(256) void k_combine(int64_t T, int d, int k,
                                                 const float* __restrict__ f,
                                                 const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w,
                                                 const float* __restrict__ ys,
                                                 void* __restrict__ y) {
  const int q = d / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * q) return;
  const int64_t t = i / q;
  const int c4 = (int)(i % q);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int64_t Tk = T * k;
  for (int j = 0; j < k; ++j) {
    const int64_t p = inv[t * k + j];
    if (p < 0 || p >= Tk) continue;  // a corrupt inverse permutation reads nothing
    const float wj = w[t * k + j];
    const float4 v = reinterpret_cast<const float4*>(f + p * d)[c4];
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  if (ys) {
    const float4 s = reinterpret_cast<const float4*>(ys + t * d)[c4];
    acc.x += s.x;
    acc.y += s.y;
    acc.z += s.z;
    acc.w += s.w;
  }
  if (kBF16Out) {
    ushort4 o;
    o.x = f32_to_bf16(acc.x);
    o.y = f32_to_bf16(acc.y);
    o.z = f32_to_bf16(acc.z);
    o.w = f32_to_bf16(acc.w);
    reinterpret_cast<ushort4*>(y)[i] = o;
  } else {
    reinterpret_cast<float4*>(y)[i] = acc;
  }
}

}  // namespace

hipError_t launch_combine(int64_t T, int d, int k, const float* f, const int32_t* inv_perm,
                          const float* w, const float* ys, void* y, bool bf16_out,
                          hipStream_t st) {
  const int64_t n = T * (d / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (bf16_out)
    hipLaunchKernelGGL(k_combine<true>, dim3(blocks), dim3(256), 0, st, T, d, k, f, inv_perm, w,
                       ys, y);
  else
    hipLaunchKernelGGL(k_combine<false>, dim3(blocks), dim3(256), 0, st, T, d, k, f, inv_perm, w,
                       ys, y);
  return hipGetLastError();
}

}  // namespace mm
