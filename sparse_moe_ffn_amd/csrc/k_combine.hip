// Weighted combine through the inverse permutation (MobileMoE close reading,
// section "Custom MoE kernel": expert outputs are scattered back to token
// order, weighted by the gate).  Written as a gather so that no two threads
// write the same output and no atomics are needed:
//   y[t][c] = fma(w[t][k-1], f[inv[t*k+k-1]][c], ... fma(w[t][0], f[inv[t*k]][c], 0))
//             + ys[t][c]
#include "combine_row.h"
#include "common.h"
#include "launch.h"

namespace mm {
namespace {

// One wave per token: the token's k sorted positions and gate weights are
// read once and broadcast across the wave; lane l handles the float4 columns
// l, l + 64, ... (kC4 of them).  The gathers of up to four expert rows and the
// shared row are all issued before the first sum, so a wave waits for memory
// about once per four experts.
constexpr int kMaxC4 = 8;  // float4 columns per lane: d <= 2048

// kNorm: also y_norm = y / sqrt(mean(y^2) + eps) (FP32 y only): the input of
// the next layer in a decoder stack, from the row the wave already holds.
template <int kC4, bool kBF16Out, bool kNorm>
__global__ __launch_bounds__(256) void k_combine(int64_t T, int d, int k,
                                                 const float* __restrict__ f,
                                                 const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w,
                                                 const float* __restrict__ ys,
                                                 void* __restrict__ y,
                                                 float* __restrict__ y_norm, float eps) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  combine_token<kC4, kBF16Out, kNorm>(t, T, d, k, f, inv, w, ys, y, y_norm, eps, nullptr);
}

template <int kC4>
void launch_combine_c4(int64_t T, int d, int k, const float* f, const int32_t* inv_perm,
                       const float* w, const float* ys, void* y, bool bf16_out, hipStream_t st,
                       float* y_norm, float eps) {
  const unsigned blocks = (unsigned)((T + 3) / 4);
  if (y_norm)
    hipLaunchKernelGGL((k_combine<kC4, false, true>), dim3(blocks), dim3(256), 0, st, T, d, k, f,
                       inv_perm, w, ys, y, y_norm, eps);
  else if (bf16_out)
    hipLaunchKernelGGL((k_combine<kC4, true, false>), dim3(blocks), dim3(256), 0, st, T, d, k, f,
                       inv_perm, w, ys, y, nullptr, 0.0f);
  else
    hipLaunchKernelGGL((k_combine<kC4, false, false>), dim3(blocks), dim3(256), 0, st, T, d, k, f,
                       inv_perm, w, ys, y, nullptr, 0.0f);
}

// Wider rows: one thread per (token, float4 column).
template <bool kBF16Out>
__global__ __launch_bounds__(256) void k_combine_wide(int64_t T, int d, int k,
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
                          hipStream_t st, float* y_norm, float eps) {
  if (d / 4 <= 64 * kMaxC4) {
    switch ((d / 4 + 63) / 64) {
      case 1: launch_combine_c4<1>(T, d, k, f, inv_perm, w, ys, y, bf16_out, st, y_norm, eps); break;
      case 2: launch_combine_c4<2>(T, d, k, f, inv_perm, w, ys, y, bf16_out, st, y_norm, eps); break;
      case 3: launch_combine_c4<3>(T, d, k, f, inv_perm, w, ys, y, bf16_out, st, y_norm, eps); break;
      case 4: launch_combine_c4<4>(T, d, k, f, inv_perm, w, ys, y, bf16_out, st, y_norm, eps); break;
      case 5: launch_combine_c4<5>(T, d, k, f, inv_perm, w, ys, y, bf16_out, st, y_norm, eps); break;
      case 6: launch_combine_c4<6>(T, d, k, f, inv_perm, w, ys, y, bf16_out, st, y_norm, eps); break;
      case 7: launch_combine_c4<7>(T, d, k, f, inv_perm, w, ys, y, bf16_out, st, y_norm, eps); break;
      default: launch_combine_c4<8>(T, d, k, f, inv_perm, w, ys, y, bf16_out, st, y_norm, eps); break;
    }
  } else {
    const unsigned blocks = (unsigned)((T * (d / 4) + 255) / 256);
    if (bf16_out)
      hipLaunchKernelGGL(k_combine_wide<true>, dim3(blocks), dim3(256), 0, st, T, d, k, f, inv_perm,
                         w, ys, y);
    else
      hipLaunchKernelGGL(k_combine_wide<false>, dim3(blocks), dim3(256), 0, st, T, d, k, f,
                         inv_perm, w, ys, y);
    if (y_norm) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_rmsnorm(T, d, eps, static_cast<const float*>(y), y_norm, st);
    }
  }
  return hipGetLastError();
}

}  // namespace mm
